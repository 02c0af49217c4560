// Device numerics for the NVFP4 kernels on gfx950 (CDNA4).
//
// E2M1 elements, E4M3FN block scales and an FP32 tensor scale, as the NVFP4
// format is described in "Coder390 NVFP4 校正（校准）方式" §2 (format
// paragraph) and "NVFP4 量化流程说明" §2.2 / §5.4.
//
// Exact E2M1 rounding without a per-element divide
// ------------------------------------------------
// For a block scale d the exact rule is: index = number of midpoints m_k
// (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) that |x|/d passes, where "passes" is
// |x| > m_k d for midpoints whose upper neighbour has an odd index and
// |x| >= m_k d otherwise (round to nearest, ties to even), saturating at 6.
//
// The fast path computes y = x * r with r ~ 1/d in fp32 and lets the gfx950
// FP4 convert (v_cvt_scalef32_pk_fp4_f32 with a unit scale: round to nearest
// even, saturating, sign of zero kept) pick the code.  y is monotone in x, so
// for a given d the fast path agrees with the exact rule for EVERY bf16 input
// iff it agrees on the two bf16 values adjacent to each exact boundary m_k d.
// cert_code() checks exactly those 14 inputs once per code and table build;
// codes that fail (rare) use the exact threshold path tau_k, which compares
// |x| against precomputed fp32 "strict" thresholds equivalent to the exact
// comparison for every fp32 x.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kBlock = 16;
constexpr int kCodes = 127;          // finite non-negative E4M3FN codes 0x00..0x7E

// E2M1 midpoints between neighbouring magnitudes and whether a tie rounds up.
__device__ __forceinline__ float e2m1_mid(int k) {
  const float m[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  return m[k];
}
__device__ __forceinline__ bool e2m1_tie_up(int k) { return (k & 1) != 0; }   // upper index k+1 even

// Value of an E4M3FN code 0..126 (exact).
__host__ __device__ __forceinline__ float e4m3_value(int c) {
  int e = c >> 3, m = c & 7;
  return e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), e - 10);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> two FP4 codes in byte `sel` of `old` (element a in the low nibble).
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}
// Byte `sel` of `src` (two FP4 codes) -> two exact fp32 values.
template <int SEL>
__device__ __forceinline__ void fp4x2_to_f32(uint32_t src, float& a, float& b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  f2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(src, 1.0f, SEL);
  a = v.x; b = v.y;
}

// Fast-path magnitude index of one value (used for certification only).
__device__ __forceinline__ int fast_index(float x, float r) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x * r, 0.0f, 1.0f, 0);
  return (int)(w & 7u);
}

// Largest bf16 pattern whose value is <= B (B >= 0, exact double).
__device__ __forceinline__ uint32_t bf16_floor_pattern(double B) {
  if (!(B < 3.3895313892515355e38)) return 0x7F7Fu;             // >= max finite bf16
  float f = __double2float_rz(B);
  return __float_as_uint(f) >> 16;                                // truncation = round down
}

__device__ __forceinline__ double bf16_pattern_value(uint32_t p) {
  return (double)__uint_as_float(p << 16);
}

// Per-code constants of one tensor scale, built once per workgroup.
struct CodeTables {
  float d[128];          // RN_f32(e4m3(c) * scale_2); d[127] = 0
  float r[128];          // fast-path reciprocal (0 for d == 0)
  float tau[128][8];     // exact strict thresholds for the slow path
  uint32_t cert[4];      // bit c set: fast path exact for code c
};

// Strict fp32 threshold tau with (|x| > tau) == (|x| passes m*d) for all fp32 x.
__device__ __forceinline__ float strict_threshold(float m, float d, bool tie_up) {
  double P = (double)m * (double)d;            // exact
  float p = (float)P;                          // nearest
  double pd = (double)p;
  bool exact = (pd == P);
  float rd = (pd > P) ? __uint_as_float(__float_as_uint(p) - 1u) : p;   // round down
  if (exact && tie_up && p > 0.0f) rd = __uint_as_float(__float_as_uint(p) - 1u);
  return rd;
}

// Does the fast path reproduce the exact rule for every bf16 input at (d, r)?
__device__ __forceinline__ bool cert_code(float d, float r) {
  if (d == 0.0f) return true;                  // r = 0: every code has magnitude 0
  if (!(r < 3.0e38f)) return false;
  for (int k = 0; k < 7; ++k) {
    double B = (double)e2m1_mid(k) * (double)d;
    uint32_t b0 = bf16_floor_pattern(B);
    bool at = bf16_pattern_value(b0) == B;
    uint32_t xp = (at && e2m1_tie_up(k)) ? b0 : b0 + 1u;   // smallest bf16 passing m_k
    if (xp <= 0x7F7Fu) {
      if (fast_index(__uint_as_float(xp << 16), r) < k + 1) return false;
    }
    if (xp >= 1u) {
      uint32_t xm = xp - 1u;
      if (xm > 0x7F7Fu) xm = 0x7F7Fu;
      if (fast_index(__uint_as_float(xm << 16), r) > k) return false;
    }
  }
  return true;
}

// Fill the tables for scale_2 = s2 (call with all threads; syncs inside).
// force_exact != 0 marks every code uncertified (exact path only; a test hook).
__device__ inline void build_code_tables(CodeTables& t, float s2, int force_exact) {
  int c = threadIdx.x;
  if (c < 4) t.cert[c] = 0u;
  __syncthreads();
  if (c < 128) {
    float d = 0.0f, r = 0.0f;
    if (c < kCodes) {
      d = (float)((double)e4m3_value(c) * (double)s2);
      r = (d == 0.0f) ? 0.0f : 1.0f / d;
    }
    t.d[c] = d;
    t.r[c] = r;
    for (int k = 0; k < 7; ++k) t.tau[c][k] = (d == 0.0f) ? __builtin_inff() : strict_threshold(e2m1_mid(k), d, e2m1_tie_up(k));
    t.tau[c][7] = __builtin_inff();
    bool ok = !force_exact && (c < kCodes) && cert_code(d, r);
    if (ok) atomicOr(&t.cert[c >> 5], 1u << (c & 31));
  }
  __syncthreads();
}

__device__ __forceinline__ bool is_cert(const CodeTables& t, int c) {
  return (t.cert[c >> 5] >> (c & 31)) & 1u;
}

// Exact magnitude index of |x| with the code's strict thresholds.
__device__ __forceinline__ int exact_index(float ax, const float* tau) {
  int idx = 0;
#pragma unroll
  for (int k = 0; k < 7; ++k) idx += (ax > tau[k]) ? 1 : 0;
  return idx;
}

// Signed E2M1 magnitude for an index 0..7.
__device__ __forceinline__ float e2m1_mag(int idx) {
  const float g[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  return g[idx];
}

}  // namespace nvfp4
