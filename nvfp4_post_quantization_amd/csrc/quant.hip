// Tensor amax -> scale_2, the dynamic per-16 NVFP4 quantizer, and the
// two-DequantizeLinear chain.  All three are single HBM passes.
//
// scale_2 = amax / (6 * 448) ("NVFP4 量化流程说明" §3.4), computed as the
// page writes it, in double and then stored as FP32 (that equals the correctly
// rounded FP32 quotient for every FP32 amax, since 2688 = 21 * 2^7 keeps the
// exact quotient away from FP32 rounding midpoints).
//
// Dynamic quantizer ("NVFP4 量化流程说明" §3.4-§3.5): one lane per 16-element
// block.  The block code RNE(amax_b / (6 scale_2)) is found exactly by a
// binary search over 126 bf16-pattern thresholds (one per E4M3 midpoint);
// the elements are then quantized with the certified fast path or the exact
// threshold path (nvfp4_device.hpp).
//
// Dequant ("NVFP4 量化流程说明" §5.4): DQ1 d = RN_f32(e4m3 * scale_2),
// DQ2 RN_f32(e2m1 * d), cast to BF16 (v_cvt_pk_bf16_f32, nearest even).
#include "common.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- amax ----

__global__ void amax_init_kernel(uint32_t* acc) {
  if (threadIdx.x == 0) *acc = 0u;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

// Per-WG maximum of |x| as a bf16 magnitude pattern, published with one
// atomicMax on the fp32 bit pattern (non-negative floats order like uints).
__device__ __forceinline__ void publish_max(uint32_t m, uint32_t* acc) {
  __shared__ uint32_t part[8];
  m = wave_max(m);
  int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) part[w] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) r = max(r, part[i]);
    if (r) atomicMax(acc, r << 16);
  }
}

__device__ __forceinline__ uint32_t absmax_word(uint32_t m, uint32_t v) {
  m = max(m, v & 0x7FFFu);
  return max(m, (v >> 16) & 0x7FFFu);
}

__global__ __launch_bounds__(256) void amax_reduce_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                          uint32_t* acc) {
  const uint4* x16 = reinterpret_cast<const uint4*>(x);
  const int64_t n16 = n >> 3;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t m = 0;
  int64_t i = gid;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    uint4 a = x16[i], b = x16[i + stride], c = x16[i + 2 * stride], d = x16[i + 3 * stride];
    m = absmax_word(m, a.x); m = absmax_word(m, a.y); m = absmax_word(m, a.z); m = absmax_word(m, a.w);
    m = absmax_word(m, b.x); m = absmax_word(m, b.y); m = absmax_word(m, b.z); m = absmax_word(m, b.w);
    m = absmax_word(m, c.x); m = absmax_word(m, c.y); m = absmax_word(m, c.z); m = absmax_word(m, c.w);
    m = absmax_word(m, d.x); m = absmax_word(m, d.y); m = absmax_word(m, d.z); m = absmax_word(m, d.w);
  }
  for (; i < n16; i += stride) {
    uint4 a = x16[i];
    m = absmax_word(m, a.x); m = absmax_word(m, a.y); m = absmax_word(m, a.z); m = absmax_word(m, a.w);
  }
  if (gid < n - (n16 << 3)) m = max(m, (uint32_t)x[(n16 << 3) + gid] & 0x7FFFu);
  publish_max(m, acc);
}

__global__ void amax_finalize_kernel(const uint32_t* acc, float* scale2_out, float* amax_out) {
  if (threadIdx.x == 0) {
    float amax = __uint_as_float(*acc);
    float s2 = (float)((double)amax / 6.0 / 448.0);
    if (amax_out) *amax_out = amax;
    *scale2_out = s2;
  }
}

int launch_compute_scale2(const uint16_t* x, int64_t n, float* scale2_out, float* amax_out, hipStream_t s) {
  uint32_t* acc = reinterpret_cast<uint32_t*>(amax_out ? amax_out : scale2_out);
  amax_init_kernel<<<1, 64, 0, s>>>(acc);
  int st = launch_status("amax_init_kernel");
  if (st) return st;
  if (n > 0) {
    int64_t n16 = n >> 3;
    int64_t want = (n16 + 255) / 256;
    int grid = (int)(want < kStreamGrid ? (want > 0 ? want : 1) : kStreamGrid);
    amax_reduce_kernel<<<grid, 256, 0, s>>>(x, n, acc);
    st = launch_status("amax_reduce_kernel");
    if (st) return st;
  }
  amax_finalize_kernel<<<1, 64, 0, s>>>(acc, scale2_out, amax_out);
  return launch_status("amax_finalize_kernel");
}

// ------------------------------------------------------ dynamic quantizer ----

// Quantize 8 words (16 bf16) at code c; returns the two packed dwords.
__device__ __forceinline__ uint2 quantize_block(const uint32_t* wv, int c, const CodeTables& t) {
  uint2 out;
  const float r = t.r[c];
  if (is_cert(t, c)) {
    uint32_t lo = 0, hi = 0;
    lo = cvt_fp4x2<0>(lo, bf16lo(wv[0]) * r, bf16hi(wv[0]) * r);
    lo = cvt_fp4x2<1>(lo, bf16lo(wv[1]) * r, bf16hi(wv[1]) * r);
    lo = cvt_fp4x2<2>(lo, bf16lo(wv[2]) * r, bf16hi(wv[2]) * r);
    lo = cvt_fp4x2<3>(lo, bf16lo(wv[3]) * r, bf16hi(wv[3]) * r);
    hi = cvt_fp4x2<0>(hi, bf16lo(wv[4]) * r, bf16hi(wv[4]) * r);
    hi = cvt_fp4x2<1>(hi, bf16lo(wv[5]) * r, bf16hi(wv[5]) * r);
    hi = cvt_fp4x2<2>(hi, bf16lo(wv[6]) * r, bf16hi(wv[6]) * r);
    hi = cvt_fp4x2<3>(hi, bf16lo(wv[7]) * r, bf16hi(wv[7]) * r);
    out.x = lo; out.y = hi;
  } else if (is_cert2(t, c)) {
    const float rh = t.rh[c], rl = t.rl[c], d = t.d[c];
    uint32_t o[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float a = quot1(bf16lo(wv[i]), d, rh, rl), b = quot1(bf16hi(wv[i]), d, rh, rl);
      const uint32_t byte = cvt_fp4x2<0>(0u, a, b) & 0xFFu;
      o[i >> 2] |= byte << (8 * (i & 3));
    }
    out.x = o[0]; out.y = o[1];
  } else {
    uint32_t o[2] = {0u, 0u};
    for (int e = 0; e < 16; ++e) {
      uint32_t bits = (wv[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
      float ax = __uint_as_float((bits & 0x7FFFu) << 16);
      uint32_t nib = (uint32_t)exact_index(ax, t.tau[c]) | ((bits >> 12) & 8u);
      o[e >> 3] |= nib << ((e & 7) * 4);
    }
    out.x = o[0]; out.y = o[1];
  }
  return out;
}

__global__ __launch_bounds__(256) void quantize_dynamic_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                               int64_t k, int64_t ldx,
                                                               const float* __restrict__ scale2,
                                                               uint8_t* __restrict__ packed,
                                                               uint8_t* __restrict__ codes, int force_exact) {
  __shared__ CodeTables t;
  __shared__ int32_t tp[128];
  const float s2 = *scale2;
  build_code_search(tp, s2);
  build_code_tables(t, s2, force_exact);    // syncs
  const int64_t nb = k >> 4;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= nb) return;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const uint4* src = reinterpret_cast<const uint4*>(x + r * ldx + g * 16);
    uint4 v0 = src[0], v1 = src[1];
    uint32_t wv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t P = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) P = absmax_word(P, wv[i]);
    int c = block_code(P, tp, s2);
    uint2 q = quantize_block(wv, c, t);
    *reinterpret_cast<uint2*>(packed + r * (k >> 1) + g * 8) = q;
    codes[r * nb + g] = (uint8_t)c;
  }
}

static dim3 row_block_grid(int64_t rows, int64_t nb, int64_t rows_per_wg) {
  int64_t gx = (nb + 255) / 256;
  int64_t gy = (rows + rows_per_wg - 1) / rows_per_wg;
  if (gy > 65535) gy = 65535;
  if (gy < 1) gy = 1;
  return dim3((unsigned)gx, (unsigned)gy, 1);
}

int launch_quantize_dynamic(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, const float* scale2,
                            uint8_t* packed, uint8_t* codes, hipStream_t s) {
  if (rows == 0) return NVFP4_OK;
  const int64_t nb = k >> 4;
  // enough rows per workgroup to amortise the per-workgroup code tables
  int64_t wgs_x = (nb + 255) / 256;
  int64_t rpw = (rows * wgs_x + kStreamGrid - 1) / kStreamGrid;
  if (rpw < 1) rpw = 1;
  quantize_dynamic_kernel<<<row_block_grid(rows, nb, rpw), 256, 0, s>>>(x, rows, k, ldx, scale2, packed, codes,
                                                                               force_exact_flag());
  return launch_status("quantize_dynamic_kernel");
}

// ---------------------------------------------------------------- dequant ----

__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ packed,
                                                      const uint8_t* __restrict__ codes,
                                                      const float* __restrict__ scale2, int64_t rows, int64_t k,
                                                      uint16_t* __restrict__ out) {
  __shared__ float dt[256];                 // E4M3FN: bit 7 = sign, 0x7F / 0xFF = NaN
  const float s2 = *scale2;
  {
    int c = threadIdx.x;
    int m = c & 0x7F;
    float v = m < kCodes ? (float)((double)e4m3_value(m) * (double)s2) : __builtin_nanf("");
    dt[c] = (c & 0x80) ? -v : v;
  }
  __syncthreads();
  const int64_t nb = k >> 4;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= nb) return;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const uint2 p = *reinterpret_cast<const uint2*>(packed + r * (k >> 1) + g * 8);
    const float d = dt[codes[r * nb + g]];
    uint32_t o[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t w = h ? p.y : p.x;
      float a0, b0, a1, b1, a2, b2, a3, b3;
      fp4x2_to_f32<0>(w, a0, b0);
      fp4x2_to_f32<1>(w, a1, b1);
      fp4x2_to_f32<2>(w, a2, b2);
      fp4x2_to_f32<3>(w, a3, b3);
      f32x2 v0 = {a0 * d, b0 * d}, v1 = {a1 * d, b1 * d}, v2 = {a2 * d, b2 * d}, v3 = {a3 * d, b3 * d};
      o[4 * h + 0] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v0, bf16x2));
      o[4 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v1, bf16x2));
      o[4 * h + 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2, bf16x2));
      o[4 * h + 3] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v3, bf16x2));
    }
    uint4* dst = reinterpret_cast<uint4*>(out + r * k + g * 16);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

int launch_dequant(const uint8_t* packed, const uint8_t* codes, const float* scale2, int64_t rows, int64_t k,
                   uint16_t* out, hipStream_t s) {
  if (rows == 0) return NVFP4_OK;
  const int64_t nb = k >> 4;
  int64_t wgs_x = (nb + 255) / 256;
  int64_t rpw = (rows * wgs_x + kStreamGrid - 1) / kStreamGrid;
  if (rpw < 1) rpw = 1;
  dequant_kernel<<<row_block_grid(rows, nb, rpw), 256, 0, s>>>(packed, codes, scale2, rows, k, out);
  return launch_status("dequant_kernel");
}

}  // namespace nvfp4
