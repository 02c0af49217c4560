// Tensor amax -> scale_2, the dynamic per-16 NVFP4 quantizer, and the
// two-DequantizeLinear chain.  All three are single HBM passes.
//
// scale_2 = amax / (6 * 448) ("NVFP4 量化流程说明" §3.4), computed as the
// page writes it, in double and then stored as FP32 (that equals the correctly
// rounded FP32 quotient for every FP32 amax, since 2688 = 21 * 2^7 keeps the
// exact quotient away from FP32 rounding midpoints).
//
// Dynamic quantizer ("NVFP4 量化流程说明" §3.4-§3.5): one lane per 16-element
// block.  The block code RNE(amax_b / (6 scale_2)) is estimated from the FP32
// quotient and made exact against 126 bf16-pattern thresholds (one per E4M3
// midpoint; binary search when 1/(6 scale_2) overflows);
// the elements are then quantized with the certified fast path or the exact
// threshold path (nvfp4_device.hpp).
//
// Fake QDQ ("NVFP4 量化流程说明" §2.2, the QuantLinear input quantizer): the
// dynamic quantizer followed by the two-DQ chain in the same lane, bf16 out.
//
// Dequant ("NVFP4 量化流程说明" §5.4): DQ1 d = RN_f32(e4m3 * scale_2),
// DQ2 RN_f32(e2m1 * d), cast to BF16 (v_cvt_pk_bf16_f32, nearest even); one
// lane per half block.
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

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// running |x| max of two bf16 lanes at once (v_pk_max_u16 on the magnitudes)
__device__ __forceinline__ u16x2 absmax2(u16x2 m, uint32_t v) {
  return __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, v) & u16x2{0x7FFF, 0x7FFF});
}

constexpr int kAmaxUnroll = 8;          // 16-byte loads in flight per thread
constexpr int kAmaxGrid = 256;          // one workgroup per CU: fewest same-address atomics (measured best)

__global__ __launch_bounds__(256) void amax_reduce_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                          uint32_t* acc) {
  const uint4* x16 = reinterpret_cast<const uint4*>(x);
  const int64_t n16 = n >> 3;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u16x2 m2 = u16x2{0, 0};
  int64_t i = gid;
  for (; i + (kAmaxUnroll - 1) * stride < n16; i += kAmaxUnroll * stride) {
    uint4 v[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) v[u] = ld_nt4(x16 + i + u * stride);
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      m2 = absmax2(m2, v[u].x); m2 = absmax2(m2, v[u].y); m2 = absmax2(m2, v[u].z); m2 = absmax2(m2, v[u].w);
    }
  }
  for (; i < n16; i += stride) {
    const uint4 v = x16[i];
    m2 = absmax2(m2, v.x); m2 = absmax2(m2, v.y); m2 = absmax2(m2, v.z); m2 = absmax2(m2, v.w);
  }
  uint32_t m = max((uint32_t)m2.x, (uint32_t)m2.y);
  if (gid < n - (n16 << 3)) m = max(m, (uint32_t)x[(n16 << 3) + gid] & 0x7FFFu);
  publish_max(m, acc);
}

// scale = amax / 6 / 448 (NVFP4 tensor scale) or amax / 448 (FP8 E4M3
// per-tensor scale), in double and then stored as FP32.
__global__ void amax_finalize_kernel(const uint32_t* acc, float* scale2_out, float* amax_out, int fp8) {
  if (threadIdx.x == 0) {
    float amax = __uint_as_float(*acc);
    float s2 = fp8 ? (float)((double)amax / 448.0) : (float)((double)amax / 6.0 / 448.0);
    if (amax_out) *amax_out = amax;
    *scale2_out = s2;
  }
}

static int launch_amax_scale(const uint16_t* x, int64_t n, float* scale2_out, float* amax_out, int fp8,
                             hipStream_t s) {
  uint32_t* acc = reinterpret_cast<uint32_t*>(amax_out ? amax_out : scale2_out);
  amax_init_kernel<<<1, 64, 0, s>>>(acc);
  int st = launch_status("amax_init_kernel");
  if (st) return st;
  if (n > 0) {
    int64_t n16 = n >> 3;
    int64_t want = (n16 + 256 * kAmaxUnroll - 1) / (256 * kAmaxUnroll);
    int grid = (int)(want < kAmaxGrid ? (want > 0 ? want : 1) : kAmaxGrid);
    amax_reduce_kernel<<<grid, 256, 0, s>>>(x, n, acc);
    st = launch_status("amax_reduce_kernel");
    if (st) return st;
  }
  amax_finalize_kernel<<<1, 64, 0, s>>>(acc, scale2_out, amax_out, fp8);
  return launch_status("amax_finalize_kernel");
}

int launch_compute_scale2(const uint16_t* x, int64_t n, float* scale2_out, float* amax_out, hipStream_t s) {
  return launch_amax_scale(x, n, scale2_out, amax_out, 0, s);
}

int launch_fp8_scale(const uint16_t* x, int64_t n, float* scale_out, float* amax_out, hipStream_t s) {
  return launch_amax_scale(x, n, scale_out, amax_out, 1, s);
}

// ------------------------------------------------------ dynamic quantizer ----

// Quantize 8 words (16 bf16) at code c; returns the two packed dwords.
__device__ __forceinline__ uint2 quantize_block(const uint32_t* wv, int c, const CodeTables& t, int mode) {
  float x[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) { x[2 * i] = bf16lo(wv[i]); x[2 * i + 1] = bf16hi(wv[i]); }
  return nibbles16(x, c, t, mode);
}

constexpr int kUnits = 4;                // blocks per thread per batch (loads in flight)
constexpr int kQuantGrid = 1024;         // quantizers: four workgroups per CU hide the E2M1 work (measured
                                         // 23.6 -> 21.0 us on [8192, 4096] against 512)
constexpr int kDequantGrid = 512;        // dequant: two per CU (1024 measured 9% slower)

// Position of flat block index u (row-major [rows][nb]) advanced by a fixed
// stride without a 64-bit division per step.
struct BlockPos {
  int64_t r, g;
  __device__ __forceinline__ void advance(int64_t dr, int64_t dg, int64_t nb) {
    r += dr;
    g += dg;
    if (g >= nb) { g -= nb; ++r; }
  }
};

// bf16 of RN_f32(e2m1 * d) for the 8 nibbles of one word (the two-DQ chain).
__device__ __forceinline__ uint4 dequant_word(uint32_t w, float d) {
  float a0, b0, a1, b1, a2, b2, a3, b3;
  fp4x2_to_f32<0>(w, a0, b0);
  fp4x2_to_f32<1>(w, a1, b1);
  fp4x2_to_f32<2>(w, a2, b2);
  fp4x2_to_f32<3>(w, a3, b3);
  const f32x2 v0 = {a0 * d, b0 * d}, v1 = {a1 * d, b1 * d}, v2 = {a2 * d, b2 * d}, v3 = {a3 * d, b3 * d};
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_convertvector(v0, bf16x2)),
                    __builtin_bit_cast(uint32_t, __builtin_convertvector(v1, bf16x2)),
                    __builtin_bit_cast(uint32_t, __builtin_convertvector(v2, bf16x2)),
                    __builtin_bit_cast(uint32_t, __builtin_convertvector(v3, bf16x2)));
}

// FQ = false: packed nibbles + block codes (the dynamic quantizer).  FQ = true:
// the fake QDQ, i.e. the same quantization followed by the two-DQ chain,
// written as bf16 [rows][ldo] without the packed intermediate.
template <bool FQ>
__global__ __launch_bounds__(256) void quantize_dynamic_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                               int64_t k, int64_t ldx,
                                                               const float* __restrict__ scale2,
                                                               uint8_t* __restrict__ packed,
                                                               uint8_t* __restrict__ codes,
                                                               uint16_t* __restrict__ out, int64_t ldo,
                                                               int force_exact) {
  __shared__ CodeTables t;
  __shared__ int32_t tp[128];
  const int64_t nb = k >> 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t dr = stride / nb, dg = stride % nb;
  const int64_t u0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  BlockPos pos{u0 / nb, u0 % nb};

  // the first batch is requested before the tables are built (it does not
  // depend on them), so the table set-up hides under the load latency
  uint4 v[kUnits][2];
  auto load = [&](BlockPos p) {
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
      if (p.r < rows) {
        const uint4* src = reinterpret_cast<const uint4*>(x + p.r * ldx + p.g * 16);
        v[j][0] = ld_nt4(src);
        v[j][1] = ld_nt4(src + 1);
      }
      p.advance(dr, dg, nb);
    }
  };
  load(pos);
  const float s2 = *scale2;
  const float inv = (float)(1.0 / (6.0 * (double)s2));
  const bool est = inv > 0.0f && inv < __builtin_inff();     // wave-uniform
  build_code_search(tp, s2);
  build_code_tables(t, s2, force_exact);    // syncs
  const int mode = table_mode(t);

  while (pos.r < rows) {
    uint32_t wv[kUnits][8];
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
      wv[j][0] = v[j][0].x; wv[j][1] = v[j][0].y; wv[j][2] = v[j][0].z; wv[j][3] = v[j][0].w;
      wv[j][4] = v[j][1].x; wv[j][5] = v[j][1].y; wv[j][6] = v[j][1].z; wv[j][7] = v[j][1].w;
    }
    BlockPos next = pos;
#pragma unroll
    for (int j = 0; j < kUnits; ++j) next.advance(dr, dg, nb);
    load(next);                              // next batch in flight while this one is quantized
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
      if (pos.r < rows) {
        u16x2 m2 = u16x2{0, 0};
#pragma unroll
        for (int i = 0; i < 8; ++i) m2 = absmax2(m2, wv[j][i]);
        const uint32_t P = max((uint32_t)m2.x, (uint32_t)m2.y);
        const int c = est ? block_code_est(P, tp, inv) : block_code(P, tp, s2);
        const uint2 q = quantize_block(wv[j], c, t, mode);
        if constexpr (FQ) {
          const float d = t.d[c];
          uint4* dst = reinterpret_cast<uint4*>(out + pos.r * ldo + pos.g * 16);
          dst[0] = dequant_word(q.x, d);
          dst[1] = dequant_word(q.y, d);
        } else {
          *reinterpret_cast<uint2*>(packed + pos.r * (k >> 1) + pos.g * 8) = q;
          codes[pos.r * nb + pos.g] = (uint8_t)c;
        }
      }
      pos.advance(dr, dg, nb);
    }
  }
}

static unsigned flat_grid(int64_t rows, int64_t nb, int64_t cap) {
  const int64_t want = (rows * nb + 256 * kUnits - 1) / (256 * kUnits);
  return (unsigned)(want < cap ? (want > 0 ? want : 1) : cap);
}

int launch_quantize_dynamic(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, const float* scale2,
                            uint8_t* packed, uint8_t* codes, hipStream_t s) {
  if (rows == 0) return NVFP4_OK;
  quantize_dynamic_kernel<false><<<flat_grid(rows, k >> 4, kQuantGrid), 256, 0, s>>>(x, rows, k, ldx, scale2, packed, codes,
                                                                         nullptr, 0, force_exact_flag());
  return launch_status("quantize_dynamic_kernel");
}

int launch_fakequant(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, const float* scale2, uint16_t* out,
                     int64_t ldo, hipStream_t s) {
  if (rows == 0) return NVFP4_OK;
  quantize_dynamic_kernel<true><<<flat_grid(rows, k >> 4, kQuantGrid), 256, 0, s>>>(x, rows, k, ldx, scale2, nullptr, nullptr,
                                                                        out, ldo, force_exact_flag());
  return launch_status("fakequant_kernel");
}

// ---------------------------------------------------------------- dequant ----

// One lane per half block (8 elements): a 4-byte nibble load and one 16-byte
// bf16 store, so each wave instruction covers one contiguous run.
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ packed,
                                                      const uint8_t* __restrict__ codes,
                                                      const float* __restrict__ scale2, int64_t rows, int64_t k,
                                                      uint16_t* __restrict__ out) {
  __shared__ float dt[256];                 // E4M3FN: bit 7 = sign, 0x7F / 0xFF = NaN
  const int64_t nh = k >> 3;                // half blocks per row
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t dr = stride / nh, dg = stride % nh;
  const int64_t u0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  BlockPos pos{u0 / nh, u0 % nh};
  uint32_t p[kUnits];
  uint32_t cd[kUnits];
  auto load = [&](BlockPos q) {
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
      if (q.r < rows) {
        p[j] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(packed + q.r * (k >> 1) + q.g * 4));
        cd[j] = codes[q.r * (k >> 4) + (q.g >> 1)];
      }
      q.advance(dr, dg, nh);
    }
  };
  load(pos);
  {
    const float s2 = *scale2;
    const int c = threadIdx.x;
    const int m = c & 0x7F;
    const float val = m < kCodes ? (float)((double)e4m3_value(m) * (double)s2) : __builtin_nanf("");
    dt[c] = (c & 0x80) ? -val : val;
  }
  __syncthreads();
  while (pos.r < rows) {
    uint32_t pc[kUnits], cc[kUnits];
#pragma unroll
    for (int j = 0; j < kUnits; ++j) { pc[j] = p[j]; cc[j] = cd[j]; }
    BlockPos next = pos;
#pragma unroll
    for (int j = 0; j < kUnits; ++j) next.advance(dr, dg, nh);
    load(next);
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
      if (pos.r < rows) {
        *reinterpret_cast<uint4*>(out + pos.r * k + pos.g * 8) = dequant_word(pc[j], dt[cc[j]]);
      }
      pos.advance(dr, dg, nh);
    }
  }
}

int launch_dequant(const uint8_t* packed, const uint8_t* codes, const float* scale2, int64_t rows, int64_t k,
                   uint16_t* out, hipStream_t s) {
  if (rows == 0) return NVFP4_OK;
  dequant_kernel<<<flat_grid(rows, k >> 3, kDequantGrid), 256, 0, s>>>(packed, codes, scale2, rows, k, out);
  return launch_status("dequant_kernel");
}

}  // namespace nvfp4
