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
// Three launches, no same-address atomics on the hot path (device-scope
// atomics serialise per address on this part):
//  (1) partial maxima of the E8M0 bytes: workgroup x of group g folds the
//      chunks x, x + nx, ... of its group and stores its maximum valid code
//      (int16, -1 = none) at codes[g][2x] (the group's codes region is
//      rewritten by pass 3, so it serves as scratch);
//  (2) one thread per group: k_max from the nx partials, scale_2 =
//      2^(k_max - 8) (2^-8 when the group has no valid exponent), fallback
//      count 0;
//  (3) codes for every MX block, with the workgroup's fallback blocks
//      requantized together at its end (one atomic add per workgroup for the
//      fallback count).
#include "common.hpp"
#include "nvfp4_device.hpp"


namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
static_assert(kThreads == 256, "the code table of pass 3 takes one entry per thread");

constexpr int kKmaxWgs = 4096;                          // pass-1 workgroups, spread over the groups
constexpr int kCodesWgs = 2048;                         // pass-3 workgroups, spread over the groups
constexpr int kKmaxLoads = 8;                          // 16-byte loads in flight per thread in pass 1
constexpr int64_t kKmaxChunk = 16 * kThreads * kKmaxLoads;   // E8M0 bytes per workgroup step
constexpr int kCodesSub = 4;                            // 8-byte exponent loads per thread per pass-3 step
constexpr int64_t kCodesChunk = 8 * kThreads * kCodesSub;    // MX blocks per workgroup step

// Largest valid code (!= 255) among 16 E8M0 bytes, or -1.
__device__ __forceinline__ int32_t max_valid16(const uint4& v) {
  const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
  uint32_t mm = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    mm = max(mm, max(max(wds[i] & 0xFFu, (wds[i] >> 8) & 0xFFu), max((wds[i] >> 16) & 0xFFu, wds[i] >> 24)));
  if (mm != 0xFFu) return (int32_t)mm;
  int32_t r = -1;                                       // a NaN exponent: redo without it
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t b = (wds[i >> 2] >> (8 * (i & 3))) & 0xFFu;
    if (b != 0xFFu) r = max(r, (int32_t)b);
  }
  return r;
}

// Pass 1: workgroup (x, g) folds chunks x, x + nx, ... of group g (16-byte
// loads where the chunk is 16-aligned and whole, bytes otherwise) and stores
// its maximum valid code at partial[g * stride16 + x].  Ordinary (cached)
// loads here: measured on the MoE expert set, MALL defeated, 109.7 us for the
// cast against 112.1 us with non-temporal ones (pass 3 keeps non-temporal
// loads: cached ones there measured 121-127 us).
__global__ __launch_bounds__(kThreads) void cast_kmax_kernel(const uint8_t* __restrict__ e8m0, int64_t per_group,
                                                             int16_t* __restrict__ partial, int64_t stride16) {
  const int64_t g = blockIdx.y;
  const int64_t nx = gridDim.x;
  const uint8_t* e = e8m0 + g * per_group;
  const bool aligned = ((reinterpret_cast<uintptr_t>(e) & 15u) == 0);
  int32_t m = -1;
  for (int64_t c0 = (int64_t)blockIdx.x * kKmaxChunk; c0 < per_group; c0 += nx * kKmaxChunk) {
    if (aligned && c0 + kKmaxChunk <= per_group) {
      uint4 v[kKmaxLoads];
#pragma unroll
      for (int u = 0; u < kKmaxLoads; ++u) v[u] = *reinterpret_cast<const uint4*>(e + c0 + 16 * (threadIdx.x + kThreads * u));
#pragma unroll
      for (int u = 0; u < kKmaxLoads; ++u) m = max(m, max_valid16(v[u]));
    } else {
      const int64_t c1 = c0 + kKmaxChunk < per_group ? c0 + kKmaxChunk : per_group;
      for (int64_t q = c0 + threadIdx.x; q < c1; q += kThreads) {
        const int32_t b = e[q];
        if (b != 0xFF) m = max(m, b);
      }
    }
  }
  __shared__ int32_t part[kThreads / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t r = -1;
    for (int i = 0; i < kThreads / 64; ++i) r = max(r, part[i]);
    partial[g * stride16 + blockIdx.x] = (int16_t)r;
  }
}

// Pass 2: one thread per group.
__global__ void cast_scale_kernel(const int16_t* __restrict__ partial, int64_t stride16, int64_t nx,
                                  int64_t groups, float* __restrict__ scale2, int64_t* fallback) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= groups) return;
  int32_t m = -1;
  for (int64_t x = 0; x < nx; ++x) m = max(m, (int32_t)partial[g * stride16 + x]);
  const int32_t km = m >= 0 ? m : 127;                  // no valid exponent: k_max taken as 0
  scale2[g] = ldexpf(1.0f, km - 127 - 8);
  if (fallback) fallback[g] = 0;
}

// E4M3 code of 2^e for e in [-9, 8].
__device__ __forceinline__ uint32_t pow2_code(int e) {
  return e >= -6 ? (uint32_t)((e + 7) << 3) : (uint32_t)(1 << (e + 9));
}

// Requantize one fallback MX block (its 16 bytes of nibbles in v) at
// delta = k_max - k_j > 17; writes the new nibbles to nib16 if any half is
// nonzero and returns the two E4M3 codes (low byte = first half).
__device__ __forceinline__ uint32_t fallback_requant(uint4 v, int delta, uint8_t* nib16) {
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

// Pass 3: workgroup (x, g) takes steps x, x + nx, ... of group g.  Where the
// step is 8-aligned and whole, a thread codes kCodesSub runs of 8 consecutive
// MX blocks, kThreads * 8 blocks apart (per run one 8-byte E8M0 load and one
// 16-byte code store, so each wave instruction covers one contiguous span),
// with the next step's exponents loaded before the current step is coded:
// 32-64 bytes of loads in flight per thread (measured: with one run per step
// the pass was latency-bound).  Other steps go block by block.  The code pair
// of an E8M0 byte depends only on it and the group's k_max, so the workgroup
// first tabulates all 256 bytes in LDS (entries of blocks outside the
// window carry kFbFlag).  Codes go out with non-temporal stores (measured on MI355X: 139 ->
// 115 us for the MoE expert set, MALL defeated; fewer workgroups were slower).
// Fallback blocks are rare and scattered.  Their table entry is the usual
// fallback code pair 0x0101, stored as a placeholder, with a flag in bit 31
// (dropped when the pairs are packed); a lane whose run has a flagged entry
// appends those blocks to a list in LDS;
// after its last step the workgroup requantizes the whole list at once, each
// thread taking one block with every nibble load issued before the first is
// used (measured: per-lane handling inside the steps, even deferred by one
// step, cost about 50 us of the pass on the MoE expert set).  Only a block
// with an all-zero half needs its codes patched.  Blocks beyond the list's
// capacity (not seen with realistic exponents) are handled at once.
constexpr uint32_t kFbFlag = 0x80000000u;
constexpr uint32_t kFbEntry = kFbFlag | 0x0101u;
constexpr int kFbCap = 2048;                            // fallback blocks listed per workgroup

__global__ __launch_bounds__(kThreads) void cast_codes_kernel(uint8_t* __restrict__ packed,
                                                              const uint8_t* __restrict__ e8m0,
                                                              int64_t per_group, const float* __restrict__ scale2,
                                                              uint8_t* __restrict__ codes,
                                                              unsigned long long* fallback) {
  __shared__ uint32_t tab[256];
  __shared__ uint32_t fb_j[kFbCap];                     // block index within the group
  __shared__ uint8_t fb_d[kFbCap];                      // its delta = k_max - k_j
  __shared__ uint32_t fb_n;
  __shared__ int part[kThreads / 64];
  const int64_t g = blockIdx.y;
  const int64_t nx = gridDim.x;
  // scale_2 = 2^(km - 135): km from its exponent field, or from the position
  // of its single bit when subnormal (km <= 8)
  const uint32_t sb = __float_as_uint(scale2[g]);
  const int32_t km = sb >= (1u << 23) ? (int32_t)(sb >> 23) + 8 : 17 - (int32_t)__builtin_clz(sb);
  {
    const int b = threadIdx.x;                          // kThreads == 256: one entry each
    uint32_t t;
    if (b == 0xFF) t = 0x7F7Fu;
    else if (km - b <= 17) { const uint32_t c = pow2_code(8 - (km - b)); t = c | (c << 8); }
    else t = kFbEntry;
    tab[b] = t;
  }
  if (threadIdx.x == 0) fb_n = 0u;
  __syncthreads();
  const int64_t base = g * per_group;
  const bool aligned = ((reinterpret_cast<uintptr_t>(e8m0 + base) & 7u) == 0);
  const int64_t step = nx * kCodesChunk;
  int nfb = 0;
  // a fallback block: listed, or (list full) requantized here
  const bool listable = per_group <= 0xFFFFFFFFll;       // list entries hold 32-bit block indices
  auto fallback_block_at = [&](int64_t jg, int delta) {
    const uint32_t slot = listable ? atomicAdd(&fb_n, 1u) : (uint32_t)kFbCap;
    if (slot < (uint32_t)kFbCap) {
      fb_j[slot] = (uint32_t)(jg - base);
      fb_d[slot] = (uint8_t)delta;
    } else {
      const uint32_t cc = fallback_requant(*reinterpret_cast<const uint4*>(packed + jg * 16), delta, packed + jg * 16);
      if (cc != 0x0101u) *reinterpret_cast<uint16_t*>(codes + 2 * jg) = (uint16_t)cc;
      ++nfb;
    }
  };
  int64_t c0 = (int64_t)blockIdx.x * kCodesChunk;
  auto whole = [&](int64_t c) { return aligned && c + kCodesChunk <= per_group; };
  // sub-step u of a step: 8 consecutive blocks per thread at c + 8 * (threadIdx.x + kThreads * u)
  uint2 e[kCodesSub];
  auto load_step = [&](int64_t c) {
#pragma unroll
    for (int u = 0; u < kCodesSub; ++u) e[u] = ld_nt2(e8m0 + base + c + 8 * (threadIdx.x + kThreads * u));
  };
  if (c0 < per_group && whole(c0)) load_step(c0);
  for (; c0 < per_group; c0 += step) {
    if (whole(c0)) {
      uint2 cur[kCodesSub];
#pragma unroll
      for (int u = 0; u < kCodesSub; ++u) cur[u] = e[u];
      const int64_t n0 = c0 + step;
      if (n0 < per_group && whole(n0)) load_step(n0);
#pragma unroll
      for (int u = 0; u < kCodesSub; ++u) {
        const int64_t j = base + c0 + 8 * (threadIdx.x + kThreads * u);
        const uint32_t ew[2] = {cur[u].x, cur[u].y};
        uint32_t cw[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) cw[i] = tab[(ew[i >> 2] >> (8 * (i & 3))) & 0xFFu];
        // pairs of code pairs: low halves of two entries (drops the flag)
        st_nt4(codes + 2 * j, make_uint4(__builtin_amdgcn_perm(cw[1], cw[0], 0x05040100u),
                                         __builtin_amdgcn_perm(cw[3], cw[2], 0x05040100u),
                                         __builtin_amdgcn_perm(cw[5], cw[4], 0x05040100u),
                                         __builtin_amdgcn_perm(cw[7], cw[6], 0x05040100u)));
        const uint32_t flags = cw[0] | cw[1] | cw[2] | cw[3] | cw[4] | cw[5] | cw[6] | cw[7];
        if (flags & kFbFlag) {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (cw[i] & kFbFlag) fallback_block_at(j + i, km - (int32_t)((ew[i >> 2] >> (8 * (i & 3))) & 0xFFu));
        }
      }
    } else {
      const int64_t c1 = c0 + kCodesChunk < per_group ? c0 + kCodesChunk : per_group;
      for (int64_t u = c0 + threadIdx.x; u < c1; u += kThreads) {
        const int64_t j = base + u;
        const uint32_t b = e8m0[j];
        const uint32_t cc = tab[b];
        if (cc & kFbFlag) fallback_block_at(j, km - (int32_t)b);
        codes[2 * j] = (uint8_t)(cc & 0xFFu);
        codes[2 * j + 1] = (uint8_t)(cc >> 8);
      }
    }
  }
  // the listed fallback blocks, four per thread per round, loads first
  __syncthreads();
  const int nl = (int)(fb_n < (uint32_t)kFbCap ? fb_n : (uint32_t)kFbCap);
  for (int r0 = 0; r0 < nl; r0 += 4 * kThreads) {
    uint4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int s = r0 + q * kThreads + threadIdx.x;
      if (s < nl) v[q] = *reinterpret_cast<const uint4*>(packed + (base + fb_j[s]) * 16);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int s = r0 + q * kThreads + threadIdx.x;
      if (s < nl) {
        const int64_t jg = base + fb_j[s];
        const uint32_t cc = fallback_requant(v[q], (int)fb_d[s], packed + jg * 16);
        if (cc != 0x0101u) *reinterpret_cast<uint16_t*>(codes + 2 * jg) = (uint16_t)cc;
        ++nfb;
      }
    }
  }
  if (fallback) {
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

}  // namespace

int launch_mx_cast(uint8_t* packed, const uint8_t* e8m0, int64_t groups, int64_t mats, int64_t rows, int64_t k,
                   uint8_t* codes, float* scale2, int64_t* fallback, hipStream_t s) {
  const int64_t per_group = mats * rows * (k / 32);   // MX blocks (= E8M0 bytes) per group; k % 32 == 0
  // workgroups per group: about kCodesWgs (kKmaxWgs) in all, at most one per step; the
  // pass-1 partials (int16, one per workgroup) fit in the group's 2*per_group
  // code bytes since nx <= per_group
  if (per_group == 0) {                               // no rows: scale_2 = 2^-8, no fallback blocks
    cast_scale_kernel<<<(unsigned)((groups + 255) / 256), 256, 0, s>>>(nullptr, 0, 0, groups, scale2, fallback);
    return launch_status("cast_scale_kernel");
  }
  const int64_t want1 = (kKmaxWgs + groups - 1) / groups;
  const int64_t want3 = (kCodesWgs + groups - 1) / groups;
  int64_t nx1 = (per_group + kKmaxChunk - 1) / kKmaxChunk;
  if (nx1 > want1) nx1 = want1;
  int64_t nx3 = (per_group + kCodesChunk - 1) / kCodesChunk;
  if (nx3 > want3) nx3 = want3;
  int16_t* partial = reinterpret_cast<int16_t*>(codes);
  const int64_t stride16 = per_group;                 // int16 slots per group = 2*per_group bytes
  int st;
  // grid.y is limited to 65535: run the groups in batches
  for (int64_t g0 = 0; g0 < groups; g0 += 65535) {
    const int64_t ng = (groups - g0 < 65535) ? groups - g0 : 65535;
    cast_kmax_kernel<<<dim3((unsigned)nx1, (unsigned)ng, 1), kThreads, 0, s>>>(e8m0 + g0 * per_group, per_group,
                                                                               partial + g0 * stride16, stride16);
    if ((st = launch_status("cast_kmax_kernel"))) return st;
  }
  cast_scale_kernel<<<(unsigned)((groups + 255) / 256), 256, 0, s>>>(partial, stride16, nx1, groups, scale2,
                                                                     fallback);
  if ((st = launch_status("cast_scale_kernel"))) return st;
  for (int64_t g0 = 0; g0 < groups; g0 += 65535) {
    const int64_t ng = (groups - g0 < 65535) ? groups - g0 : 65535;
    cast_codes_kernel<<<dim3((unsigned)nx3, (unsigned)ng, 1), kThreads, 0, s>>>(
        packed + g0 * per_group * 16, e8m0 + g0 * per_group, per_group, scale2 + g0, codes + g0 * per_group * 2,
        fallback ? reinterpret_cast<unsigned long long*>(fallback + g0) : nullptr);
    if ((st = launch_status("cast_codes_kernel"))) return st;
  }
  return NVFP4_OK;
}

}  // namespace nvfp4
