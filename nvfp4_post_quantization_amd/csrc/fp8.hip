// FP8 E4M3 tier with per-tensor static scales: the W8A8 attention layers of
// the mixed W4A4+W8A8 tier ("Coder390 NVFP4 校正（校准）方式" §3, layer table;
// the FP8 activation scales are static, gathered in calibration).
//
//   s    = RN_f32(amax / 448)                      (fp8e4m3_compute_scale)
//   code = E4M3FN RNE_sat(x / s), exact quotient, sign kept   (fp8e4m3_quantize)
//   out  = RN_bf16(RN_f32(e4m3(code) * s))          (fp8e4m3_dequant)
//
// Quantize.  gfx950's v_cvt_pk_fp8_f32 rounds fp32 to E4M3FN to nearest even
// and is exact up to 464; above it returns NaN instead of saturating, so its
// input is clamped to +-448 first (every value in (448, 464] rounds to 448
// anyway).  It is applied to y = x * r for a reciprocal r of s that each
// workgroup certifies once: x -> code is monotone in the bf16 pattern, so it
// is the exact map for every bf16 input iff it puts the two patterns around
// each of the 126 code thresholds on the right sides.  Candidates are RN(1/s)
// and its neighbours up to 4 ulps away.  Without a certified r (s = 0, 1/s
// overflowing, or the test hook NVFP4MI_FORCE_EXACT) every code comes from the
// exact thresholds: an estimate from the fp32 quotient fixed by one compare on
// each side, or a binary search when 1/s overflows.
//
// Dequant.  The hardware decode (v_cvt_pk_f32_fp8, exact for all 256 codes,
// NaN for 0x7F/0xFF), one fp32 multiply by s (correctly rounded: the exact
// product has at most 28 significant bits before rounding), then the bf16
// cast (nearest even).
#include "common.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
constexpr int kUnits = 4;            // 8-element units per lane per batch (loads in flight)
constexpr int kGrid = 512;           // two workgroups per CU
constexpr float kE4M3Max = 448.0f;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Position of flat unit index u (row-major [rows][n]) advanced by a fixed
// stride without a 64-bit division per step.
struct UnitPos {
  int64_t r, g;
  __device__ __forceinline__ void advance(int64_t dr, int64_t dg, int64_t n) {
    r += dr;
    g += dg;
    if (g >= n) { g -= n; ++r; }
  }
};

// Four codes of x * r, clamped, through the hardware convert (bytes in order).
__device__ __forceinline__ uint32_t fast4(uint32_t w0, uint32_t w1, float r) {
  const float a = __builtin_amdgcn_fmed3f(bf16lo(w0) * r, -kE4M3Max, kE4M3Max);
  const float b = __builtin_amdgcn_fmed3f(bf16hi(w0) * r, -kE4M3Max, kE4M3Max);
  const float c = __builtin_amdgcn_fmed3f(bf16lo(w1) * r, -kE4M3Max, kE4M3Max);
  const float d = __builtin_amdgcn_fmed3f(bf16hi(w1) * r, -kE4M3Max, kE4M3Max);
  int o = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  o = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, o, true);
  return (uint32_t)o;
}

// Magnitude code of a positive bf16 pattern on the fast path.
__device__ __forceinline__ int fast_code(uint32_t P, float r) {
  const float y = __builtin_amdgcn_fmed3f(__uint_as_float(P << 16) * r, -kE4M3Max, kE4M3Max);
  return __builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false) & 0x7F;
}

// Exact code of one bf16 value (thresholds tp for S = s).
__device__ __forceinline__ uint32_t exact_code(uint32_t bits, const int32_t* tp, float s, float inv, bool est) {
  const uint32_t P = bits & 0x7FFFu;
  int c;
  if (s == 0.0f) c = P ? kCodes - 1 : 0;                       // x / 0 saturates
  else if (est) c = max(e4m3_code_est_raw(P, tp, inv), 0);
  else c = e4m3_code_search(P, tp);
  return (uint32_t)c | ((bits >> 8) & 0x80u);
}

__device__ __forceinline__ uint32_t exact4(uint32_t w0, uint32_t w1, const int32_t* tp, float s, float inv, bool est) {
  return exact_code(w0 & 0xFFFFu, tp, s, inv, est) | (exact_code(w0 >> 16, tp, s, inv, est) << 8) |
         (exact_code(w1 & 0xFFFFu, tp, s, inv, est) << 16) | (exact_code(w1 >> 16, tp, s, inv, est) << 24);
}

__global__ __launch_bounds__(kThreads) void fp8_quantize_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                                 int64_t k, int64_t ldx,
                                                                 const float* __restrict__ scale,
                                                                 uint8_t* __restrict__ q, int force_exact) {
  __shared__ int32_t tp[128];
  __shared__ float r_cert;
  const int64_t n = k >> 3;                                   // units per row
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t dr = stride / n, dg = stride % n;
  const int64_t u0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  UnitPos pos{u0 / n, u0 % n};

  // first batch in flight while the thresholds are built and r certified
  uint4 v[kUnits];
  auto load = [&](UnitPos p) {
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
      if (p.r < rows) v[j] = ld_nt4(x + p.r * ldx + p.g * 8);
      p.advance(dr, dg, n);
    }
  };
  load(pos);

  const float s = *scale;
  const float inv = (float)(1.0 / (double)s);
  const bool est = inv > 0.0f && inv < __builtin_inff();
  build_e4m3_thresholds(tp, (double)s);
  if (threadIdx.x == 0) r_cert = 0.0f;
  __syncthreads();
  if (est && force_exact == 0) {
    const int b = threadIdx.x;                                 // boundary between codes b and b+1
    for (int i = 0; i < 9; ++i) {
      const int delta = (i & 1) ? -((i + 1) >> 1) : (i >> 1);
      const float r = __uint_as_float(__float_as_uint(inv) + (uint32_t)delta);
      bool ok = r < __builtin_inff();                         // uniform
      if (ok && b < kCodes - 1) {
        const int32_t t = tp[b];                               // >= 0 for s > 0
        if (t + 1 <= 0x7F7F) ok = ok && fast_code((uint32_t)(t + 1), r) >= b + 1;
        ok = ok && fast_code((uint32_t)t, r) <= b;
      }
      if (__syncthreads_and(ok)) {
        if (threadIdx.x == 0) r_cert = r;
        break;
      }
    }
    __syncthreads();
  }
  const float r = r_cert;                                      // 0: no certified reciprocal
  const bool fast = r != 0.0f;

  while (pos.r < rows) {
    uint4 cur[kUnits];
#pragma unroll
    for (int j = 0; j < kUnits; ++j) cur[j] = v[j];
    UnitPos next = pos;
#pragma unroll
    for (int j = 0; j < kUnits; ++j) next.advance(dr, dg, n);
    load(next);
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
      if (pos.r < rows) {
        uint2 o;
        if (fast) {
          o.x = fast4(cur[j].x, cur[j].y, r);
          o.y = fast4(cur[j].z, cur[j].w, r);
        } else {
          o.x = exact4(cur[j].x, cur[j].y, tp, s, inv, est);
          o.y = exact4(cur[j].z, cur[j].w, tp, s, inv, est);
        }
        *reinterpret_cast<uint2*>(q + pos.r * k + pos.g * 8) = o;
      }
      pos.advance(dr, dg, n);
    }
  }
}

template <bool HI>
__device__ __forceinline__ uint32_t dequant2(uint32_t w, float s) {
  const f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  const f32x2 y = {f.x * s, f.y * s};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(y, bf16x2));
}

__global__ __launch_bounds__(kThreads) void fp8_dequant_kernel(const uint8_t* __restrict__ q,
                                                               const float* __restrict__ scale, int64_t rows,
                                                               int64_t k, uint16_t* __restrict__ out) {
  const int64_t n = k >> 3;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t dr = stride / n, dg = stride % n;
  const int64_t u0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  UnitPos pos{u0 / n, u0 % n};
  uint2 v[kUnits];
  auto load = [&](UnitPos p) {
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
      if (p.r < rows) v[j] = ld_nt2(q + p.r * k + p.g * 8);
      p.advance(dr, dg, n);
    }
  };
  load(pos);
  const float s = *scale;
  while (pos.r < rows) {
    uint2 cur[kUnits];
#pragma unroll
    for (int j = 0; j < kUnits; ++j) cur[j] = v[j];
    UnitPos next = pos;
#pragma unroll
    for (int j = 0; j < kUnits; ++j) next.advance(dr, dg, n);
    load(next);
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
      if (pos.r < rows) {
        *reinterpret_cast<uint4*>(out + pos.r * k + pos.g * 8) =
            make_uint4(dequant2<false>(cur[j].x, s), dequant2<true>(cur[j].x, s), dequant2<false>(cur[j].y, s),
                       dequant2<true>(cur[j].y, s));
      }
      pos.advance(dr, dg, n);
    }
  }
}

unsigned grid_for(int64_t rows, int64_t n) {
  const int64_t want = (rows * n + kThreads * kUnits - 1) / (kThreads * kUnits);
  return (unsigned)(want < kGrid ? (want > 0 ? want : 1) : kGrid);
}

}  // namespace

int launch_fp8_quantize(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, const float* scale, uint8_t* q,
                        hipStream_t s) {
  fp8_quantize_kernel<<<grid_for(rows, k >> 3), kThreads, 0, s>>>(x, rows, k, ldx, scale, q, force_exact_flag());
  return launch_status("fp8_quantize_kernel");
}

int launch_fp8_dequant(const uint8_t* q, const float* scale, int64_t rows, int64_t k, uint16_t* out, hipStream_t s) {
  fp8_dequant_kernel<<<grid_for(rows, k >> 3), kThreads, 0, s>>>(q, scale, rows, k, out);
  return launch_status("fp8_dequant_kernel");
}

}  // namespace nvfp4
