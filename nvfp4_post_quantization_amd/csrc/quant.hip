// Tensor amax -> scale_2 (one tensor, or up to kScaleBatch tensors in the
// same three launches), the dynamic per-16 NVFP4 quantizer, and the
// two-DequantizeLinear chain.  All three are single HBM passes.
//
// scale_2 = amax / (6 * 448) ("NVFP4 量化流程说明" §3.4), computed as the
// page writes it, in double and then stored as FP32 (that equals the correctly
// rounded FP32 quotient for every FP32 amax, since 2688 = 21 * 2^7 keeps the
// exact quotient away from FP32 rounding midpoints).
//
// Dynamic quantizer ("NVFP4 量化流程说明" §3.4-§3.5): one lane per 16-element
// block (for rows of whole 64-block units, the blocks reach their lanes
// through contiguous 1 KiB wave loads and one DPP exchange of half blocks).
// The block code RNE(amax_b / (6 scale_2)) is estimated from the FP32
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
// lane per block of a 64-block unit for rows of whole units, else one lane
// per half block.
#include <type_traits>

#include "common.hpp"
#include "nvfp4_device.hpp"


namespace nvfp4 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- amax ----

// Up to kScaleBatch tensors per launch: workgroup w takes its grid-stride
// share of tensor 0, then of tensor 1, ..., so no workgroup idles at a
// tensor boundary; one atomicMax per workgroup and tensor.  acc[t] is
// amax_out[t] when given, else scale2_out[t] (both FP32 arrays of count).
struct AmaxBatch {
  const uint16_t* x[kScaleBatch];
  int64_t n[kScaleBatch];
  uint32_t* acc[kScaleBatch];
  float* scale_out[kScaleBatch];
  float* amax_out[kScaleBatch];
  int count;
  int fp8;
};

__global__ void amax_init_kernel(const AmaxBatch b) {
  if ((int)threadIdx.x < b.count) *b.acc[threadIdx.x] = 0u;
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
  __syncthreads();                       // the previous tensor's reads of part are done
  if ((threadIdx.x & 63) == 0) part[w] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) r = max(r, part[i]);
    if (r) atomicMax(acc, r << 16);
  }
}

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// running |x| max of two bf16 lanes at once (v_pk_max_u16 on the magnitudes)
__device__ __forceinline__ u16x2 absmax2(u16x2 m, uint32_t v) {
  return __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, v) & u16x2{0x7FFF, 0x7FFF});
}

constexpr int kAmaxUnroll = 8;          // 16-byte loads in flight per thread
constexpr int kAmaxGrid = 256;          // one workgroup per CU: fewest same-address atomics (measured best)

__global__ __launch_bounds__(256) void amax_reduce_kernel(const AmaxBatch b) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int t = 0; t < b.count; ++t) {
    const uint16_t* __restrict__ x = b.x[t];
    const int64_t n = b.n[t];
    const uint4* x16 = reinterpret_cast<const uint4*>(x);
    const int64_t n16 = n >> 3;
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
    publish_max(m, b.acc[t]);
  }
}

// scale = amax / 6 / 448 (NVFP4 tensor scale) or amax / 448 (FP8 E4M3
// per-tensor scale), in double and then stored as FP32.
__global__ void amax_finalize_kernel(const AmaxBatch b) {
  const int t = threadIdx.x;
  if (t < b.count) {
    float amax = __uint_as_float(*b.acc[t]);
    float s2 = b.fp8 ? (float)((double)amax / 448.0) : (float)((double)amax / 6.0 / 448.0);
    if (b.amax_out[t]) *b.amax_out[t] = amax;
    *b.scale_out[t] = s2;
  }
}

static int launch_amax_batch(const uint16_t* const* xs, const int64_t* ns, int count, float* scale_out,
                             float* amax_out, int fp8, hipStream_t s) {
  AmaxBatch b{};
  b.count = count;
  b.fp8 = fp8;
  int64_t most = 0;
  for (int t = 0; t < count; ++t) {
    b.x[t] = xs[t];
    b.n[t] = ns[t];
    b.scale_out[t] = scale_out + t;
    b.amax_out[t] = amax_out ? amax_out + t : nullptr;
    b.acc[t] = reinterpret_cast<uint32_t*>(amax_out ? amax_out + t : scale_out + t);
    if (ns[t] > most) most = ns[t];
  }
  amax_init_kernel<<<1, 64, 0, s>>>(b);
  int st = launch_status("amax_init_kernel");
  if (st) return st;
  if (most > 0) {
    const int64_t want = ((most >> 3) + 256 * kAmaxUnroll - 1) / (256 * kAmaxUnroll);
    const int grid = (int)(want < kAmaxGrid ? (want > 0 ? want : 1) : kAmaxGrid);
    amax_reduce_kernel<<<grid, 256, 0, s>>>(b);
    st = launch_status("amax_reduce_kernel");
    if (st) return st;
  }
  amax_finalize_kernel<<<1, 64, 0, s>>>(b);
  return launch_status("amax_finalize_kernel");
}

int launch_compute_scale2(const uint16_t* x, int64_t n, float* scale2_out, float* amax_out, hipStream_t s) {
  return launch_amax_batch(&x, &n, 1, scale2_out, amax_out, 0, s);
}

int launch_compute_scale2_batch(const uint16_t* const* xs, const int64_t* ns, int count, float* scale2_out,
                                float* amax_out, hipStream_t s) {
  return launch_amax_batch(xs, ns, count, scale2_out, amax_out, 0, s);
}

int launch_fp8_scale(const uint16_t* x, int64_t n, float* scale_out, float* amax_out, hipStream_t s) {
  return launch_amax_batch(&x, &n, 1, scale_out, amax_out, 1, s);
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
constexpr int kDequantGrid = 512;        // half-block dequant: two per CU (1024 measured 9% slower)

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
  build_all_tables(tp, t, s2, force_exact);    // syncs
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
          st_nt2(packed + pos.r * (k >> 1) + pos.g * 8, q);
          st_nt1(codes + pos.r * nb + pos.g, (uint8_t)c);
        }
      }
      pos.advance(dr, dg, nb);
    }
  }
}

// Rows made of whole 64-block units (k a multiple of 1024): a wave takes one
// unit (2 KiB of bf16) per step with two contiguous 1 KiB loads, so every
// load instruction fills whole cache lines (the one-lane-per-block loads
// above read 16 bytes at a 32-byte stride: two instructions per line, and
// measured 17.4 us of pure loading on [8192, 4096] against 11.5 us for a
// plain read).  After the loads lane l holds half l % 2 of block l / 2 of
// the first KiB (a) and of block 32 + l / 2 of the second (b); adjacent lanes
// swap one half (DPP quad_perm 1,0,3,2), so that even lane 2j owns block j
// and odd lane 2j + 1 owns block 32 + j, and from there each lane quantizes
// its own block exactly as above.  A wave works on kPairUnits units per step
// with the next two steps' loads in flight.
constexpr int kPairUnits = 2;

__device__ __forceinline__ uint32_t swap_pair(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
}

template <bool FQ>
__global__ __launch_bounds__(256) void quantize_units_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                             int64_t k, int64_t ldx,
                                                             const float* __restrict__ scale2,
                                                             uint8_t* __restrict__ packed,
                                                             uint8_t* __restrict__ codes,
                                                             uint16_t* __restrict__ out, int64_t ldo,
                                                             int force_exact) {
  __shared__ CodeTables t;
  __shared__ int32_t tp[128];
  const int lane = threadIdx.x & 63;
  const int64_t nb = k >> 4;
  const int64_t upr = nb >> 6;                               // units per row
  const int64_t units = rows * upr;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  int64_t u0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const bool odd = lane & 1;
  const int bi = odd ? 32 + (lane >> 1) : (lane >> 1);      // the block this lane owns after the swap

  // two register sets, each holding kPairUnits units: the loop works on one
  // while the other's loads are in flight, so two iterations of loads (and
  // four units at the start, issued before the tables are built) are in
  // flight per wave
  uint4 a[2][kPairUnits], b[2][kPairUnits];
  auto load = [&](int set, int64_t u) {
#pragma unroll
    for (int q = 0; q < kPairUnits; ++q) {
      const int64_t uq = u + q * nwaves;
      if (uq < units) {
        const int64_t r = uq / upr;
        const uint4* src = reinterpret_cast<const uint4*>(x + r * ldx + (uq - r * upr) * 1024);
        a[set][q] = ld_nt4(src + lane);
        b[set][q] = ld_nt4(src + 64 + lane);
      }
    }
  };
  const int64_t step = kPairUnits * nwaves;
  load(0, u0);                                               // before the tables: hides their set-up
  load(1, u0 + step);
  const float s2 = *scale2;
  const float inv = (float)(1.0 / (6.0 * (double)s2));
  const bool est = inv > 0.0f && inv < __builtin_inff();     // wave-uniform
  build_all_tables(tp, t, s2, force_exact);                     // syncs
  const int mode_rt = table_mode(t);

  // one copy of the loop per E2M1 mode (uniform over the launch), so the
  // common modes run branch-free per block
  auto run = [&](auto mode_c) {
    constexpr int mode = decltype(mode_c)::value;
    auto process = [&](int set, int64_t u) {
      uint32_t wv[kPairUnits][8];
#pragma unroll
      for (int q = 0; q < kPairUnits; ++q) {
        const uint4 send = odd ? a[set][q] : b[set][q];
        const uint4 recv = make_uint4(swap_pair(send.x), swap_pair(send.y), swap_pair(send.z), swap_pair(send.w));
        const uint4 lo = odd ? recv : a[set][q], hi = odd ? b[set][q] : recv;
        wv[q][0] = lo.x; wv[q][1] = lo.y; wv[q][2] = lo.z; wv[q][3] = lo.w;
        wv[q][4] = hi.x; wv[q][5] = hi.y; wv[q][6] = hi.z; wv[q][7] = hi.w;
      }
      load(set, u + 2 * step);                               // this set's next units in flight meanwhile
#pragma unroll
      for (int q = 0; q < kPairUnits; ++q) {
        const int64_t uq = u + q * nwaves;
        if (uq < units) {
          u16x2 m2 = u16x2{0, 0};
#pragma unroll
          for (int i = 0; i < 8; ++i) m2 = absmax2(m2, wv[q][i]);
          const uint32_t P = max((uint32_t)m2.x, (uint32_t)m2.y);
          const int c = est ? block_code_est(P, tp, inv) : block_code(P, tp, s2);
          const uint2 qn = quantize_block(wv[q], c, t, mode);
          const int64_t r = uq / upr;
          const int64_t g = (uq - r * upr) * 64 + bi;        // block within the row
          if constexpr (FQ) {
            const float d = t.d[c];
            uint4* dst = reinterpret_cast<uint4*>(out + r * ldo + g * 16);
            dst[0] = dequant_word(qn.x, d);
            dst[1] = dequant_word(qn.y, d);
          } else {
            st_nt2(packed + r * (k >> 1) + g * 8, qn);
            st_nt1(codes + r * nb + g, (uint8_t)c);
          }
        }
      }
    };
    for (; u0 < units; u0 += 2 * step) {
      process(0, u0);
      if (u0 + step < units) process(1, u0 + step);
    }
  };
  if (mode_rt == 0) run(std::integral_constant<int, 0>{});
  else if (mode_rt == 1) run(std::integral_constant<int, 1>{});
  else run(std::integral_constant<int, 2>{});
}

static unsigned flat_grid(int64_t rows, int64_t nb, int64_t cap) {
  const int64_t want = (rows * nb + 256 * kUnits - 1) / (256 * kUnits);
  return (unsigned)(want < cap ? (want > 0 ? want : 1) : cap);
}

// grid of the unit kernel: about kUnitGrid workgroups, fewer for small inputs.
// Three per CU: with two register sets of loads in flight the kernel takes
// 146 VGPRs, so three waves fit per SIMD (measured on [8192, 4096], MALL
// defeated: 19.1 us at 768 against 22.3 us at 1024 and 20.3 us at 512; the
// one-set loop at 1024 took 19.5 us; bounding it to 128 VGPRs spilled).
constexpr int kUnitGrid = 768;
static unsigned unit_grid(int64_t rows, int64_t k) {
  const int64_t units = rows * ((k >> 4) >> 6);
  const int64_t want = (units + 4 * kPairUnits - 1) / (4 * kPairUnits);
  return (unsigned)(want < kUnitGrid ? (want > 0 ? want : 1) : kUnitGrid);
}

int launch_quantize_dynamic(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, const float* scale2,
                            uint8_t* packed, uint8_t* codes, hipStream_t s) {
  if (rows == 0) return NVFP4_OK;
  if (((k >> 4) & 63) == 0) {
    quantize_units_kernel<false><<<unit_grid(rows, k), 256, 0, s>>>(x, rows, k, ldx, scale2, packed, codes, nullptr, 0,
                                                                    force_exact_flag());
    return launch_status("quantize_units_kernel");
  }
  quantize_dynamic_kernel<false><<<flat_grid(rows, k >> 4, kQuantGrid), 256, 0, s>>>(x, rows, k, ldx, scale2, packed, codes,
                                                                         nullptr, 0, force_exact_flag());
  return launch_status("quantize_dynamic_kernel");
}

int launch_fakequant(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, const float* scale2, uint16_t* out,
                     int64_t ldo, hipStream_t s) {
  if (rows == 0) return NVFP4_OK;
  if (((k >> 4) & 63) == 0) {
    quantize_units_kernel<true><<<unit_grid(rows, k), 256, 0, s>>>(x, rows, k, ldx, scale2, nullptr, nullptr, out, ldo,
                                                                   force_exact_flag());
    return launch_status("fakequant_units_kernel");
  }
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
        st_nt4(out + pos.r * k + pos.g * 8, dequant_word(pc[j], dt[cc[j]]));
      }
      pos.advance(dr, dg, nh);
    }
  }
}

// Rows made of whole 64-block units (k a multiple of 1024): a wave takes one
// unit per step, even lane 2j block j and odd lane 2j + 1 block 32 + j (8
// bytes of nibbles and one code each, two spans of 256 bytes per load
// instruction).  Each lane decodes both halves of its block; adjacent lanes
// swap one half (DPP quad_perm 1,0,3,2) so that the unit's 2 KiB of bf16 go
// out as two contiguous 1 KiB stores, lane l writing elements 8l..8l+7 of
// each (the one-lane-per-half-block kernel above reads 4 bytes per lane).
// The next kDqUnits units are loaded while a wave decodes its current ones
// (measured on [8192, 4096], MALL defeated: 17.6 us with 4 against 17.8 us
// with 2 and 18.3 us for the half-block kernel; 1024 workgroups were slower).
constexpr int kDqUnits = 4;
constexpr int kDqGrid = 512;

__global__ __launch_bounds__(256) void dequant_units_kernel(const uint8_t* __restrict__ packed,
                                                            const uint8_t* __restrict__ codes,
                                                            const float* __restrict__ scale2, int64_t rows,
                                                            int64_t k, uint16_t* __restrict__ out) {
  __shared__ float dt[256];                 // E4M3FN: bit 7 = sign, 0x7F / 0xFF = NaN
  const int lane = threadIdx.x & 63;
  const bool odd = lane & 1;
  const int blk = odd ? 32 + (lane >> 1) : (lane >> 1);
  const int64_t upr = k >> 10;              // units per row
  const int64_t units = rows * upr;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  int64_t u0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  uint2 nib[kDqUnits];
  uint32_t cd[kDqUnits];
  auto load = [&](int64_t u) {
#pragma unroll
    for (int q = 0; q < kDqUnits; ++q) {
      const int64_t uq = u + q * nwaves;
      if (uq < units) {
        const int64_t r = uq / upr, ui = uq - r * upr;
        nib[q] = ld_nt2(packed + r * (k >> 1) + ui * 512 + blk * 8);
        cd[q] = codes[r * (k >> 4) + ui * 64 + blk];
      }
    }
  };
  load(u0);
  {
    const float s2 = *scale2;
    const int c = threadIdx.x;
    const int m = c & 0x7F;
    const float val = m < kCodes ? (float)((double)e4m3_value(m) * (double)s2) : __builtin_nanf("");
    dt[c] = (c & 0x80) ? -val : val;
  }
  __syncthreads();
  for (; u0 < units; u0 += kDqUnits * nwaves) {
    uint2 pn[kDqUnits];
    uint32_t pc[kDqUnits];
#pragma unroll
    for (int q = 0; q < kDqUnits; ++q) { pn[q] = nib[q]; pc[q] = cd[q]; }
    load(u0 + kDqUnits * nwaves);
#pragma unroll
    for (int q = 0; q < kDqUnits; ++q) {
      const int64_t uq = u0 + q * nwaves;
      if (uq < units) {
        const float d = dt[pc[q]];
        const uint4 h0 = dequant_word(pn[q].x, d), h1 = dequant_word(pn[q].y, d);
        const uint4 send = odd ? h0 : h1;
        const uint4 recv = make_uint4(swap_pair(send.x), swap_pair(send.y), swap_pair(send.z), swap_pair(send.w));
        const int64_t r = uq / upr, ui = uq - r * upr;
        uint16_t* o = out + r * k + ui * 1024 + lane * 8;
        st_nt4(o, odd ? recv : h0);
        st_nt4(o + 512, odd ? h1 : recv);
      }
    }
  }
}

int launch_dequant(const uint8_t* packed, const uint8_t* codes, const float* scale2, int64_t rows, int64_t k,
                   uint16_t* out, hipStream_t s) {
  if (rows == 0) return NVFP4_OK;
  if ((k & 1023) == 0) {
    const int64_t units = rows * (k >> 10);
    const int64_t want = (units + 4 * kDqUnits - 1) / (4 * kDqUnits);
    const unsigned grid = (unsigned)(want < kDqGrid ? want : kDqGrid);
    dequant_units_kernel<<<grid, 256, 0, s>>>(packed, codes, scale2, rows, k, out);
    return launch_status("dequant_units_kernel");
  }
  dequant_kernel<<<flat_grid(rows, k >> 3, kDequantGrid), 256, 0, s>>>(packed, codes, scale2, rows, k, out);
  return launch_status("dequant_kernel");
}

}  // namespace nvfp4
