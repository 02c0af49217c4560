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
// Level 0 (fast path): y = x * r with a per-code fp32 r ~ 1/d, and the gfx950
// FP4 convert (v_cvt_scalef32_pk_fp4_f32 with a unit scale: round to nearest
// even, saturating, sign of zero kept) picks the code.  y is monotone in x, so
// for a given d the fast path agrees with the exact rule for EVERY bf16 input
// iff it agrees on the two bf16 values adjacent to each exact boundary m_k d.
// cert_code() checks exactly those 14 inputs when the tables are built, for
// r = RN(1/d) and its neighbours up to 4 ulps away, and keeps the first r
// that passes.  (2688 = 2^7 * 3 * 7, so for many tensor scales some m_k d
// fall within one fp32 rounding of a bf16 value; a shifted r usually still
// separates them.)
// Level 1: the quotient from a two-float reciprocal (error < 0.5 ulp + 2^-46),
// moved one ulp toward the exact value (sign of x - y d from an fma, exact):
// an fp32 y within one ulp of x/d can only sit on a midpoint when it is
// there exactly, so the convert then sees the correct side of every
// midpoint and exact ties keep the convert's ties-to-even.  Certified too.
// Level 2 (never seen in practice): compare |x| with precomputed fp32
// "strict" thresholds tau_k equivalent to the exact comparison for every
// fp32 x.
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

// Non-temporal loads for data read exactly once (streamed inputs): they keep
// it from displacing cached data.
typedef uint32_t ntu32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t ntu32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_nt4(const void* p) {
  const ntu32x4 v = __builtin_nontemporal_load(reinterpret_cast<const ntu32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_nt2(const void* p) {
  const ntu32x2 v = __builtin_nontemporal_load(reinterpret_cast<const ntu32x2*>(p));
  return make_uint2(v.x, v.y);
}
// Non-temporal stores (streamed output that nothing reads back soon).  They
// pay off where one wave store instruction covers a contiguous span (16, 8 or
// 1 bytes per lane, lanes adjacent); measured on MI355X, kernels whose lanes
// write 32 bytes each as two interleaved 16-byte stores ran up to twice as
// slow with them, so those keep ordinary stores.
__device__ __forceinline__ void st_nt4(void* p, uint4 v) {
  const ntu32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<ntu32x4*>(p));
}
__device__ __forceinline__ void st_nt2(void* p, uint2 v) {
  const ntu32x2 w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<ntu32x2*>(p));
}
__device__ __forceinline__ void st_nt1(uint8_t* p, uint8_t v) { __builtin_nontemporal_store(v, p); }

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

// The low part x * rl of a two-float quotient, clamped to the finite range
// (one v_med3).  |rl| <= 2^-24 |rh|, so x * rl overflows only when |x * rh|
// exceeds 2^24 times the largest float; the fma then still overflows, or
// stays far above the E2M1 range, with the sign of x, and the quotient
// saturates as it should, whatever the sign of rl.  Finite values pass
// unchanged.
__device__ __forceinline__ float quot_low(float x, float rl) {
  return __builtin_amdgcn_fmed3f(x * rl, -3.40282347e38f, 3.40282347e38f);
}

// Level-1 quotient: x / d from the two-float reciprocal (rh + rl ~ 1/d),
// moved one ulp toward the exact quotient when it is not exact.
__device__ __forceinline__ float quot1(float x, float d, float rh, float rl) {
  const float y = __builtin_fmaf(x, rh, quot_low(x, rl));
  const float rho = __builtin_fmaf(-y, d, x);            // x - y*d, sign exact
  const int dir = (rho > 0.0f) - (rho < 0.0f);
  uint32_t b = __float_as_uint(y);
  b += (b >> 31) ? (uint32_t)(-dir) : (uint32_t)dir;     // toward the exact value
  return __uint_as_float(b);
}

// Level-1 quotient: x / d from the two-float reciprocal, one rounding, no
// correction.
__device__ __forceinline__ float quot_tf(float x, float rh, float rl) {
  return __builtin_fmaf(x, rh, quot_low(x, rl));
}

// Fast quotient of one level: 0 = x * r (r = rh), 1 = quot_tf, 2 = quot1.
__device__ __forceinline__ float fast_quot(float x, float d, float rh, float rl, int level) {
  return level == 0 ? x * rh : (level == 1 ? quot_tf(x, rh, rl) : quot1(x, d, rh, rl));
}

// Magnitude index of one value on a fast level.
__device__ __forceinline__ int fast_index(float x, float d, float rh, float rl, int level) {
  const float y = fast_quot(x, d, rh, rl, level);
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y, 0.0f, 1.0f, 0);
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
  float r[128];          // level-0 reciprocal (0 for d == 0)
  float rh[128];         // two-float reciprocal, high part (level 1)
  float rl[128];         // two-float reciprocal, low part (level 1)
  float tau[128][8];     // exact strict thresholds (filled only for codes without a fast level)
  uint32_t cert[4];      // bit c set: level 0 (x * r) exact for code c
  uint32_t cert1[4];     // bit c set: level 1 (two-float, one rounding) exact for code c
  uint32_t cert2[4];     // bit c set: level 2 (two-float, corrected) exact for code c
  int mode;              // 0: level 0 for every code; 1: level 1 for every code; 2: per code
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

// Does the fast path reproduce the exact rule for every bf16 input at d?
__device__ __forceinline__ bool cert_code(float d, float r, float rl, int level) {
  if (d == 0.0f) return true;                  // r = 0: every code has magnitude 0
  if (!(r < 3.0e38f)) return false;
  for (int k = 0; k < 7; ++k) {
    double B = (double)e2m1_mid(k) * (double)d;
    uint32_t b0 = bf16_floor_pattern(B);
    bool at = bf16_pattern_value(b0) == B;
    uint32_t xp = (at && e2m1_tie_up(k)) ? b0 : b0 + 1u;   // smallest bf16 passing m_k
    if (xp <= 0x7F7Fu) {
      if (fast_index(__uint_as_float(xp << 16), d, r, rl, level) < k + 1) return false;
    }
    if (xp >= 1u) {
      uint32_t xm = xp - 1u;
      if (xm > 0x7F7Fu) xm = 0x7F7Fu;
      if (fast_index(__uint_as_float(xm << 16), d, r, rl, level) > k) return false;
    }
  }
  return true;
}

// Fill the tables for scale_2 = s2 (call with all threads; syncs inside).
// Levels are tried cheapest first; when every code is exact on one level, that
// level serves all codes (a uniform branch in the kernels, which matters
// since the lanes of a wave quantize at different codes).  Test hook:
// force_exact = 1 uses the exact thresholds only, 2 skips level 0, 3 skips
// levels 0 and 1.
__device__ __forceinline__ void build_code_tables(CodeTables& t, float s2, int force_exact) {
  const int c = threadIdx.x;
  if (c < 4) { t.cert[c] = 0u; t.cert1[c] = 0u; t.cert2[c] = 0u; }
  __syncthreads();
  float d = 0.0f, rh = 0.0f, rl = 0.0f;
  bool level0 = false;
  if (c < 128) {
    if (c < kCodes) {
      d = (float)((double)e4m3_value(c) * (double)s2);
      if (d != 0.0f) {
        double R = 1.0 / (double)d;
        rh = (float)R;
        rl = (float)(R - (double)rh);
      }
    }
    t.d[c] = d;
    t.rh[c] = rh;
    t.rl[c] = rl;
    float r = rh;
    if (force_exact == 0 && c < kCodes) {
      // level 0: RN(1/d), then its neighbours up to 4 ulps away
      for (int i = 0; i < 9; ++i) {
        const int delta = (i & 1) ? -((i + 1) >> 1) : (i >> 1);
        const float rt = (d == 0.0f) ? 0.0f : __uint_as_float(__float_as_uint(rh) + (uint32_t)delta);
        if (cert_code(d, rt, 0.0f, 0)) {
          r = rt;
          level0 = true;
          atomicOr(&t.cert[c >> 5], 1u << (c & 31));
          break;
        }
      }
    }
    t.r[c] = r;
  }
  __syncthreads();
  // codes 0..126 all on level 0: one uniform path, nothing else to build
  const bool all0 = t.cert[0] == ~0u && t.cert[1] == ~0u && t.cert[2] == ~0u && t.cert[3] == 0x7FFFFFFFu;
  if (all0) {
    if (c == 0) t.mode = 0;
    __syncthreads();
    return;
  }
  // level 1 for every code, so that one uniform path may serve them all
  bool level1 = false;
  if (force_exact != 1 && force_exact != 3 && c < kCodes && cert_code(d, rh, rl, 1)) {
    level1 = true;
    atomicOr(&t.cert1[c >> 5], 1u << (c & 31));
  }
  __syncthreads();
  const bool all1 = t.cert1[0] == ~0u && t.cert1[1] == ~0u && t.cert1[2] == ~0u && t.cert1[3] == 0x7FFFFFFFu;
  if (!all1 && c < 128) {
    // per-code dispatch: level 2 and the exact thresholds for codes that
    // neither cheaper level covers
    bool level2 = false;
    if (!level0 && !level1 && force_exact != 1 && c < kCodes && cert_code(d, rh, rl, 2)) {
      level2 = true;
      atomicOr(&t.cert2[c >> 5], 1u << (c & 31));
    }
    if (!level0 && !level1 && !level2) {
      for (int k = 0; k < 7; ++k) t.tau[c][k] = (d == 0.0f) ? __builtin_inff() : strict_threshold(e2m1_mid(k), d, e2m1_tie_up(k));
      t.tau[c][7] = __builtin_inff();
    }
  }
  if (c == 0) t.mode = all1 ? 1 : 2;
  __syncthreads();
}

// Fast level used for code c (3 = exact thresholds); uniform unless mode == 2.
__device__ __forceinline__ int code_level(const CodeTables& t, int c) {
  if (t.mode != 2) return t.mode;
  if ((t.cert[c >> 5] >> (c & 31)) & 1u) return 0;
  if ((t.cert1[c >> 5] >> (c & 31)) & 1u) return 1;
  if ((t.cert2[c >> 5] >> (c & 31)) & 1u) return 2;
  return 3;
}

// Exact magnitude index of |x| with the code's strict thresholds.
__device__ __forceinline__ int exact_index(float ax, const float* tau) {
  int idx = 0;
#pragma unroll
  for (int k = 0; k < 7; ++k) idx += (ax > tau[k]) ? 1 : 0;
  return idx;
}

// Packed E2M1 nibbles of 8 values (element 2i in the low nibble of byte i)
// on fast level 0-2, given the code's table values: d, its reciprocal
// (level 0: t.r, else t.rh) and t.rl; the FP4 convert (RNE, saturating) of
// the certified fast quotient.
template <int LEVEL>
__device__ __forceinline__ uint32_t nibbles8_vals(const float* x, float d, float rh, float rl) {
  static_assert(LEVEL >= 0 && LEVEL <= 2, "fast levels only");
  uint32_t nb = cvt_fp4x2<0>(0u, fast_quot(x[0], d, rh, rl, LEVEL), fast_quot(x[1], d, rh, rl, LEVEL));
  nb = cvt_fp4x2<1>(nb, fast_quot(x[2], d, rh, rl, LEVEL), fast_quot(x[3], d, rh, rl, LEVEL));
  nb = cvt_fp4x2<2>(nb, fast_quot(x[4], d, rh, rl, LEVEL), fast_quot(x[5], d, rh, rl, LEVEL));
  nb = cvt_fp4x2<3>(nb, fast_quot(x[6], d, rh, rl, LEVEL), fast_quot(x[7], d, rh, rl, LEVEL));
  return nb;
}

// Packed E2M1 nibbles of 8 values at code c on one level: levels 0-2 as
// above with the code's table values, level 3 by the exact thresholds.
template <int LEVEL>
__device__ __forceinline__ uint32_t nibbles8_level(const float* x, int c, const CodeTables& t) {
  if constexpr (LEVEL == 3) {
    const float* tau = t.tau[c];
    uint32_t o = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t nib = (uint32_t)exact_index(fabsf(x[i]), tau) | (__builtin_signbitf(x[i]) ? 8u : 0u);
      o |= nib << (i * 4);
    }
    return o;
  } else {
    return nibbles8_vals<LEVEL>(x, t.d[c], LEVEL == 0 ? t.r[c] : t.rh[c], t.rl[c]);
  }
}

// Nibbles of 8 values at code c (lane-varying).  mode = t.mode, read once
// per kernel into a scalar register: modes 0 and 1 take one level for every
// code (a uniform branch); mode 2 dispatches per code.
__device__ __forceinline__ uint32_t nibbles8(const float* x, int c, const CodeTables& t, int mode) {
  if (mode == 0) return nibbles8_level<0>(x, c, t);
  if (mode == 1) return nibbles8_level<1>(x, c, t);
  const int lvl = code_level(t, c);
  if (lvl == 0) return nibbles8_level<0>(x, c, t);
  if (lvl == 1) return nibbles8_level<1>(x, c, t);
  if (lvl == 2) return nibbles8_level<2>(x, c, t);
  return nibbles8_level<3>(x, c, t);
}

// The same for 16 values (two nibble words).
__device__ __forceinline__ uint2 nibbles16(const float* x, int c, const CodeTables& t, int mode) {
  if (mode == 0) return make_uint2(nibbles8_level<0>(x, c, t), nibbles8_level<0>(x + 8, c, t));
  if (mode == 1) return make_uint2(nibbles8_level<1>(x, c, t), nibbles8_level<1>(x + 8, c, t));
  return make_uint2(nibbles8(x, c, t, 2), nibbles8(x + 8, c, t, 2));
}

__device__ __forceinline__ int table_mode(const CodeTables& t) { return __builtin_amdgcn_readfirstlane(t.mode); }

// E2M1 magnitude for an index 0..7 ({0, .5, 1, 1.5, 2, 3, 4, 6}), table-free.
__device__ __forceinline__ float e2m1_mag(int idx) {
  const int twice = idx + max(idx - 4, 0) + 2 * max(idx - 6, 0);   // 2 * magnitude
  return 0.5f * (float)twice;
}

// Thresholds of an E4M3 encode of bf16 magnitudes over a scale S > 0:
// the code RNE_sat(|x| / S) is the number of thresholds passed, where |x|
// with bf16 pattern P passes tp[c] iff P > tp[c], tp[c] being the largest
// pattern that stays at or below the midpoint between codes c and c+1 (times
// S), ties going to the even code.  mid * S is exact in double (a midpoint has
// at most 5 significant bits, S at most 26).  tp[126] is a sentinel that no
// pattern passes (saturation at 448).
__device__ __forceinline__ void build_e4m3_thresholds(int32_t* tp, double S, int c = threadIdx.x) {
  if (c >= 0 && c < 128) {
    int32_t t = 0x7FFFFFFF;
    if (c < kCodes - 1) {
      double mid = 0.5 * ((double)e4m3_value(c) + (double)e4m3_value(c + 1));
      double M = mid * S;
      uint32_t b0 = bf16_floor_pattern(M);
      bool at = bf16_pattern_value(b0) == M;
      bool tie_up = ((c + 1) & 1) == 0;
      t = (at && tie_up) ? (int32_t)b0 - 1 : (int32_t)b0;
    }
    tp[c] = t;
  }
}

// Thresholds of the block-code search: the block code is the E4M3 encode of
// the block max over 6 * scale_2 (exact in double).
__device__ inline void build_code_search(int32_t* tp, float s2) { build_e4m3_thresholds(tp, 6.0 * (double)s2); }

// Both tables of a workgroup of at least 256 threads: the block-code
// thresholds on threads 128..255 while threads 0..127 certify the E2M1 paths
// (that certification is the longer part; run one after the other they had
// cost about 4 us at the start of every launch).  Syncs before returning.
__device__ __forceinline__ void build_all_tables(int32_t* tp, CodeTables& t, float s2, int force_exact) {
  build_e4m3_thresholds(tp, 6.0 * (double)s2, (int)threadIdx.x - 128);
  build_code_tables(t, s2, force_exact);
}

// E4M3 code estimate of pattern P over the thresholds' scale S, for
// 0 < inv = RN_f32(1 / S) < inf: the FP32 quotient P * inv is within 2^-23
// relative of the exact one, so its E4M3 rounding (computed on the bits) is
// at most one code off, and one compare on each side against the exact
// thresholds fixes it.  Written without branches so that several values'
// table reads can overlap.  For c = 0 the lower threshold read is tp[0]
// instead of "none", so the result is -1 where the exact code is 0 (P <=
// tp[0]); callers clamp.
__device__ __forceinline__ int e4m3_code_est_raw(uint32_t P, const int32_t* tp, float inv) {
  const float y = __uint_as_float(P << 16) * inv;
  const uint32_t b = __float_as_uint(y);
  const int cn = (int)((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - ((127 - 7) << 3);   // normal E4M3: 3 bits, RNE
  const int cs = (int)rintf(y * 512.0f);                                              // subnormal: k * 2^-9
  int c = y >= 0x1p-6f ? cn : cs;
  c = min(max(c, 0), kCodes - 1);
  const int32_t hi = tp[c];
  const int32_t lo = tp[max(c - 1, 0)];
  return c + ((int32_t)P > hi) - ((int32_t)P <= lo);          // thresholds increase: at most one holds
}

// Exact E4M3 code of pattern P by binary search over the thresholds (any S).
__device__ __forceinline__ int e4m3_code_search(uint32_t P, const int32_t* tp) {
  int pos = 0;
#pragma unroll
  for (int step = 64; step >= 1; step >>= 1)
    if (tp[pos + step - 1] < (int32_t)P) pos += step;
  return pos;
}

// The dynamic quantizer's block code from the block-max pattern P (tables
// from build_code_search): the E4M3 encode of P / (6 scale_2), for
// 0 < inv = RN_f32(1 / (6 scale_2)) < inf.  A nonzero block never gets scale 0
// (for c = 0 the raw estimate gives -1 or 0, both lifted by the final max).
__device__ __forceinline__ int block_code_est(uint32_t P, const int32_t* tp, float inv) {
  return max(e4m3_code_est_raw(P, tp, inv), P ? 1 : 0);
}

__device__ __forceinline__ int block_code(uint32_t P, const int32_t* tp, float s2) {
  int pos = e4m3_code_search(P, tp);
  if (s2 == 0.0f) pos = P ? (kCodes - 1) : 0;
  if (pos == 0 && P) pos = 1;                                  // nonzero block: never scale 0
  return pos;
}

}  // namespace nvfp4
