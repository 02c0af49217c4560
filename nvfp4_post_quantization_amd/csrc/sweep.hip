// Hessian-weighted E4M3 block-scale sweep (fp8_scale_sweep, "Coder390 NVFP4
// 校正（校准）方式" §2 step 3): for each 16-element weight block w of group g
// and each finite code c, cost(c) = e^T H_g e with e = w - q(c) d_c; keep the
// code of least cost (lowest code on ties).
//
// Mapping on gfx950:
//  * a workgroup owns four adjacent groups and a range of rows; wave w sweeps
//    group 4*blockIdx.x + w (H_g loaded once into registers) over those rows,
//    so the four waves read each row's 128 bytes together;
//  * the 64 lanes of a wave evaluate 16 candidate codes x 16 elements per
//    step: lane l handles code 16*tile + l%16 and elements 4*(l/16)..+3, and
//    eight tiles cover codes 0..127 (127 = NaN is skipped);
//  * e = w - q d uses the certified FP4-convert fast path for q (exact for
//    every bf16 w; uncertified codes fall back to exact thresholds);
//  * H_g e for the 16 candidates is one 16x16x16 product, four
//    v_mfma_f32_16x16x4_f32 with H_g as the A operand (lane l holds
//    H_g[l%16][4*(l/16)+s]) and the error vectors as B; the output lane holds
//    (H e)_{4*(l/16)+r} of its own candidate, so e . (H e) is a 4-term dot
//    plus two cross-row swaps (v_permlane32/16_swap); the eight tiles' MFMA
//    chains are independent and interleaved;
//  * the argmin runs per lane over its 8 codes (ascending, strict <), then
//    across the 16 candidate lanes with an explicit lowest-code tie-break.
// Costs are fp32 (the cost output is that fp32 value); nibbles are exact.
#include "common.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float exact_q(float w, const float* tau) {
  float m = e2m1_mag(exact_index(fabsf(w), tau));
  return __builtin_copysignf(m, w);
}

__device__ __forceinline__ uint32_t exact_nib(float w, const float* tau) {
  return (uint32_t)exact_index(fabsf(w), tau) | (__builtin_signbitf(w) ? 8u : 0u);
}

// Sum of v over the four 16-lane rows of the wave, identical in every lane:
// (row0 + row2) + (row1 + row3) via the gfx950 cross-row swaps.
__device__ __forceinline__ float sum_rows(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__global__ __launch_bounds__(kThreads) void sweep_kernel(const uint16_t* __restrict__ w, int64_t rows, int64_t k,
                                                         int64_t ldw, const float* __restrict__ H,
                                                         const float* __restrict__ scale2, int64_t rows_per_wg,
                                                         uint8_t* __restrict__ packed, uint8_t* __restrict__ codes,
                                                         float* __restrict__ cost, int force_exact) {
  __shared__ CodeTables t;
  const float s2 = *scale2;
  build_code_tables(t, s2, force_exact);                     // syncs; no barrier after this point

  const int64_t groups = k >> 4;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // the four waves own four adjacent groups over the same rows, so a row's
  // 4 x 32 bytes arrive as one 128-byte line
  const int64_t g = (int64_t)blockIdx.x * kWaves + wave;
  if (g >= groups) return;
  const int q = lane >> 4;
  const int cl = lane & 15;

  const float* Hg = H + g * 256;
  float hA[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) hA[s] = Hg[cl * 16 + 4 * q + s];

  float rt[8], dt[8];
  uint32_t lane_cert = 0, lane_cert2 = 0, tile_slow = 0;
#pragma unroll
  for (int tile = 0; tile < 8; ++tile) {
    const int c = 16 * tile + cl;
    rt[tile] = t.r[c];
    dt[tile] = t.d[c];
    if (c >= kCodes || is_cert(t, c)) lane_cert |= 1u << tile;
    if (c < kCodes && is_cert2(t, c)) lane_cert2 |= 1u << tile;
    uint32_t bits = (t.cert[tile >> 1] >> (16 * (tile & 1))) & 0xFFFFu;
    uint32_t need = (tile == 7) ? 0x7FFFu : 0xFFFFu;          // code 127 is not swept
    if ((bits & need) != need) tile_slow |= 1u << tile;
  }

  const int64_t r0 = (int64_t)blockIdx.y * rows_per_wg;
  int64_t r1 = r0 + rows_per_wg;
  if (r1 > rows) r1 = rows;

  for (int64_t r = r0; r < r1; ++r) {
    const uint2 wv = *reinterpret_cast<const uint2*>(w + r * ldw + g * 16 + 4 * q);
    const float w0 = bf16lo(wv.x), w1 = bf16hi(wv.x), w2 = bf16lo(wv.y), w3 = bf16hi(wv.y);
    // error vectors of all eight tiles (lane: code 16*tile + cl, elements 4q..4q+3)
    float e[8][4];
#pragma unroll
    for (int tile = 0; tile < 8; ++tile) {
      const float rr = rt[tile], dd = dt[tile];
      uint32_t nb = cvt_fp4x2<0>(0u, w0 * rr, w1 * rr);
      nb = cvt_fp4x2<1>(nb, w2 * rr, w3 * rr);
      float q0, q1, q2, q3;
      fp4x2_to_f32<0>(nb, q0, q1);
      fp4x2_to_f32<1>(nb, q2, q3);
      if (tile_slow & (1u << tile)) {                  // wave-uniform: some code of the tile uncertified
        if (!(lane_cert & (1u << tile))) {
          const int c = 16 * tile + cl;
          if (lane_cert2 & (1u << tile)) {
            const float rh = t.rh[c], rl = t.rl[c];
            uint32_t nb2 = cvt_fp4x2<0>(0u, quot1(w0, dd, rh, rl), quot1(w1, dd, rh, rl));
            nb2 = cvt_fp4x2<1>(nb2, quot1(w2, dd, rh, rl), quot1(w3, dd, rh, rl));
            fp4x2_to_f32<0>(nb2, q0, q1);
            fp4x2_to_f32<1>(nb2, q2, q3);
          } else {
            const float* tau = t.tau[c];
            q0 = exact_q(w0, tau); q1 = exact_q(w1, tau); q2 = exact_q(w2, tau); q3 = exact_q(w3, tau);
          }
        }
      }
      e[tile][0] = fmaf(-q0, dd, w0);
      e[tile][1] = fmaf(-q1, dd, w1);
      e[tile][2] = fmaf(-q2, dd, w2);
      e[tile][3] = fmaf(-q3, dd, w3);
    }
    // H e for all tiles: eight independent MFMA chains, interleaved
    floatx4 acc[8];
#pragma unroll
    for (int tile = 0; tile < 8; ++tile) acc[tile] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int tile = 0; tile < 8; ++tile)
        acc[tile] = __builtin_amdgcn_mfma_f32_16x16x4f32(hA[s], e[tile][s], acc[tile], 0, 0, 0);
    }
    float best = __builtin_inff();
    int bestc = 0;
#pragma unroll
    for (int tile = 0; tile < 8; ++tile) {
      float p = e[tile][0] * acc[tile][0];
      p = fmaf(e[tile][1], acc[tile][1], p);
      p = fmaf(e[tile][2], acc[tile][2], p);
      p = fmaf(e[tile][3], acc[tile][3], p);
      p = sum_rows(p);
      const int c = 16 * tile + cl;
      if (c < kCodes && p < best) { best = p; bestc = c; }
    }
    // argmin across the 16 candidate lanes of each row (all rows agree)
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const float ob = __shfl_xor(best, o);
      const int oc = __shfl_xor(bestc, o);
      if (ob < best || (ob == best && oc < bestc)) { best = ob; bestc = oc; }
    }
    // nibbles of this lane's 4 elements at the chosen code
    const float rr = t.r[bestc];
    uint32_t nb;
    if (is_cert(t, bestc)) {
      nb = cvt_fp4x2<0>(0u, w0 * rr, w1 * rr);
      nb = cvt_fp4x2<1>(nb, w2 * rr, w3 * rr);
    } else if (is_cert2(t, bestc)) {
      const float rh = t.rh[bestc], rl = t.rl[bestc], db = t.d[bestc];
      nb = cvt_fp4x2<0>(0u, quot1(w0, db, rh, rl), quot1(w1, db, rh, rl));
      nb = cvt_fp4x2<1>(nb, quot1(w2, db, rh, rl), quot1(w3, db, rh, rl));
    } else {
      const float* tau = t.tau[bestc];
      nb = exact_nib(w0, tau) | (exact_nib(w1, tau) << 4) | (exact_nib(w2, tau) << 8) | (exact_nib(w3, tau) << 12);
    }
    if (cl == 0) {
      *reinterpret_cast<uint16_t*>(packed + r * (k >> 1) + g * 8 + 2 * q) = (uint16_t)(nb & 0xFFFFu);
      if (q == 0) {
        codes[r * groups + g] = (uint8_t)bestc;
        if (cost) cost[r * groups + g] = best;
      }
    }
  }
}

}  // namespace

int launch_scale_sweep(const uint16_t* w, int64_t rows, int64_t k, int64_t ldw, const float* H,
                       const float* scale2, uint8_t* packed, uint8_t* codes, float* cost, hipStream_t s) {
  const int64_t groups = k >> 4;
  const int64_t gx = (groups + kWaves - 1) / kWaves;
  // about 8192 workgroups; each wave sweeps rows_per_wg blocks of its group
  int64_t rpw = (rows * gx + 8191) / 8192;
  if (rpw < 1) rpw = 1;
  int64_t chunks = (rows + rpw - 1) / rpw;
  while (chunks > 65535) {
    rpw *= 2;
    chunks = (rows + rpw - 1) / rpw;
  }
  dim3 grid((unsigned)gx, (unsigned)chunks, 1);
  sweep_kernel<<<grid, kThreads, 0, s>>>(w, rows, k, ldw, H, scale2, rpw, packed, codes, cost,
                                                     force_exact_flag());
  return launch_status("sweep_kernel");
}

}  // namespace nvfp4
