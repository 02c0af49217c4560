// Block-Hadamard rotation of the input channels under the local-Hessian
// sweep ("FP4量化技术概述：从理论到硬件实现" §3.1, MR-GPTQ: block Hadamard
// transform fused into the weights, W' = W H, activations rotated online).
// Per NVFP4 group of 16 input channels R_g = H16 / 4 (Sylvester, symmetric,
// orthogonal), so X W^T = (X R)(W R)^T and the rotated input's local Hessian
// is H'_g = R_g^T H_g R_g.
//
// nvfp4_block_hadamard: every 16-element row block x -> RN_bf16((x H16) / 4),
// computed as the Sylvester butterfly (stages h = 1, 2, 4, 8: pairs (i, i+h)
// -> (a + b, a - b)) in fp64, exact whenever the block spans less than 2^41,
// then rounded ONCE to bf16: round-to-odd to fp32 (correct for a later
// rounding to 8 bits), then the hardware cast to bf16 (nearest even).  One
// lane per block: two 16-byte loads, 64 fp64 adds, two 16-byte stores.
//
// nvfp4_hessian_hadamard: H'_g = R^T H_g R in fp64, rounded to fp32; one wave
// per group, H_g staged in LDS (so H' may overwrite H).
#include "common.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
constexpr int kUnits = 2;            // blocks in flight per lane
constexpr int kGrid = 1024;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct UnitPos {
  int64_t r, g;
  __device__ __forceinline__ void advance(int64_t dr, int64_t dg, int64_t n) {
    r += dr;
    g += dg;
    if (g >= n) { g -= n; ++r; }
  }
};

// fp64 -> fp32 rounded to odd: truncate toward zero, then set the last bit
// when inexact.  A later nearest-even rounding to bf16 (8 bits < 24 - 1) is
// then the correctly rounded bf16 of x.  Overflow truncates to the largest
// finite value, which rounds to infinity in bf16 exactly when x does.
__device__ __forceinline__ float to_f32_odd(double x) {
  const float f = (float)x;                                    // nearest
  const double d = (double)f;
  uint32_t b = __float_as_uint(f);
  if (__builtin_fabs(d) > __builtin_fabs(x)) b -= 1u;          // step back toward zero (inf -> FLT_MAX)
  if (d != x) b |= 1u;
  return __uint_as_float(b);
}

__device__ __forceinline__ uint32_t pack_bf16(double a, double b) {
  const f32x2 v = {to_f32_odd(a), to_f32_odd(b)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// (x H16) / 4 of one block, in place on v[16]
__device__ __forceinline__ void butterfly16(double* v) {
#pragma unroll
  for (int h = 1; h < 16; h *= 2) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        const double a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] *= 0.25;
}

__global__ __launch_bounds__(kThreads) void block_hadamard_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                                  int64_t k, int64_t ldx, uint16_t* out,
                                                                  int64_t ldo) {
  const int64_t n = k >> 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t dr = stride / n, dg = stride % n;
  const int64_t u0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  UnitPos pos{u0 / n, u0 % n};
  uint4 v[kUnits][2];
  auto load = [&](UnitPos p) {
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
      if (p.r < rows) {
        const uint16_t* src = x + p.r * ldx + p.g * 16;
        v[j][0] = ld_nt4(src);
        v[j][1] = ld_nt4(src + 8);
      }
      p.advance(dr, dg, n);
    }
  };
  load(pos);
  while (pos.r < rows) {
    uint32_t w[kUnits][8];
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
      w[j][0] = v[j][0].x; w[j][1] = v[j][0].y; w[j][2] = v[j][0].z; w[j][3] = v[j][0].w;
      w[j][4] = v[j][1].x; w[j][5] = v[j][1].y; w[j][6] = v[j][1].z; w[j][7] = v[j][1].w;
    }
    UnitPos next = pos;
#pragma unroll
    for (int j = 0; j < kUnits; ++j) next.advance(dr, dg, n);
    load(next);
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
      if (pos.r < rows) {
        double d[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          d[2 * i] = (double)bf16lo(w[j][i]);
          d[2 * i + 1] = (double)bf16hi(w[j][i]);
        }
        butterfly16(d);
        uint16_t* dst = out + pos.r * ldo + pos.g * 16;
        *reinterpret_cast<uint4*>(dst) = make_uint4(pack_bf16(d[0], d[1]), pack_bf16(d[2], d[3]),
                                                    pack_bf16(d[4], d[5]), pack_bf16(d[6], d[7]));
        *reinterpret_cast<uint4*>(dst + 8) = make_uint4(pack_bf16(d[8], d[9]), pack_bf16(d[10], d[11]),
                                                        pack_bf16(d[12], d[13]), pack_bf16(d[14], d[15]));
      }
      pos.advance(dr, dg, n);
    }
  }
}

// H'_g[i][j] = (1/16) sum_a sum_b s(a,i) H_g[a][b] s(b,j), s(a,i) = (-1)^popcount(a & i):
// first T = S H along one index (lane (i, b)), then along the other.
__global__ __launch_bounds__(kThreads) void hessian_hadamard_kernel(const float* H, int64_t groups, float* Hout) {
  __shared__ double T[kThreads / 64][256];
  __shared__ float Hs[kThreads / 64][256];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * (kThreads / 64) + wave;
  const bool live = g < groups;
  if (live) {
#pragma unroll
    for (int e = 0; e < 4; ++e) Hs[wave][lane + 64 * e] = H[g * 256 + lane + 64 * e];
  }
  __syncthreads();
  if (live) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = lane + 64 * e, i = idx >> 4, b = idx & 15;
      double t = 0.0;
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const double h = (double)Hs[wave][a * 16 + b];
        t = (__builtin_popcount(a & i) & 1) ? t - h : t + h;
      }
      T[wave][i * 16 + b] = t;
    }
  }
  __syncthreads();
  if (live) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = lane + 64 * e, i = idx >> 4, j = idx & 15;
      double s = 0.0;
#pragma unroll
      for (int b = 0; b < 16; ++b) {
        const double t = T[wave][i * 16 + b];
        s = (__builtin_popcount(b & j) & 1) ? s - t : s + t;
      }
      Hout[g * 256 + idx] = (float)(s * 0.0625);
    }
  }
}

}  // namespace

int launch_block_hadamard(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, uint16_t* out, int64_t ldo,
                          hipStream_t s) {
  const int64_t want = (rows * (k >> 4) + kThreads * kUnits - 1) / (kThreads * kUnits);
  const unsigned grid = (unsigned)(want < kGrid ? (want > 0 ? want : 1) : kGrid);
  block_hadamard_kernel<<<grid, kThreads, 0, s>>>(x, rows, k, ldx, out, ldo);
  return launch_status("block_hadamard_kernel");
}

int launch_hessian_hadamard(const float* H, int64_t groups, float* Hout, hipStream_t s) {
  const int64_t wgs = (groups + kThreads / 64 - 1) / (kThreads / 64);
  hessian_hadamard_kernel<<<(unsigned)wgs, kThreads, 0, s>>>(H, groups, Hout);
  return launch_status("hessian_hadamard_kernel");
}

}  // namespace nvfp4
