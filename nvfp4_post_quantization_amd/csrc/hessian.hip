// Block-diagonal local Hessian accumulation ("Coder390 NVFP4 校正（校准）方式"
// §2 step 2):  H[g] += X_g^T X_g  for every group g of 16 input channels.
//
// The work is HBM-bound (2 bytes read per element, 32 flops per element), so
// the design goal is a single coalesced pass over X:
//  * the work is cut into tiles of 64 tokens x one slab of 16 groups (256
//    channels, 512 B of every token row; 8 groups in the W4A4 variant).  A
//    grid of about two workgroups per CU takes equal contiguous ranges of the
//    slab-major tile order, so every workgroup streams the same number of
//    bytes whatever the shape;
//  * tiles go through LDS (16 B per lane, coalesced rows, non-temporal loads),
//    the next tile in flight while one is consumed (32 KiB per workgroup; the
//    W4A4 variant keeps two 16 KiB tiles in flight);
//  * H_g = X_g^T X_g is a 16x16 contraction over tokens, done with
//    v_mfma_f32_16x16x32_bf16.  In that instruction lane l supplies row l%16
//    of A and column l%16 of B for K-slots 8*(l/16)..+7; for A = X_g^T and
//    B = X_g both are "channel l%16 at 8 tokens", so one register feeds both
//    operands.  The lane's 8 tokens of one channel come from LDS by two
//    transposing reads (ds_read_b64_tr_b16); the 16-byte chunks are
//    XOR-swizzled by row so the lane groups of a read hit disjoint banks;
//  * a workgroup writes one fp32 partial per slab its range touches (at most
//    a few), one set per chunk in a chunk-list call; a second kernel adds,
//    per group, the partials of that slab's workgroups of every chunk to H in
//    fp64, in a fixed order (deterministic).
// Optionally the running max |x| (calibration step 1) is taken from the MFMA
// operands, which together hold every element of a tile.
// The W4A4 variant (nvfp4_hessian_accum_fq) accumulates the Hessian of the
// fake-quantized input instead: each lane pair quantizes its 16-element
// block in registers before the tile goes to LDS.
#include <mutex>

#include "common.hpp"
#include "nvfp4_device.hpp"

// Partial slots of nvfp4_hessian_accum_noalloc: the plain kernel's workspace
// for any shape with k <= 131072 (512 workgroups x 2 slabs x 16 groups x 1 KiB),
// held by each device that runs the library until the process ends.  Host
// code never passes this name to a kernel: it uses the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[nvfp4::kHessianScratchBytes];

namespace nvfp4 {

namespace {

// Slab geometry of SG groups (SG * 16 channels, SG * 32 bytes of a token
// row): a row is SG * 2 chunks of 16 B, one per lane, so one load pass of
// 256 threads covers kLoadRows rows and a 64-token tile takes kUnits passes;
// each of the 4 waves owns SG / 4 groups of the slab.
template <int SG>
struct Slab {
  static constexpr int kGroups = SG;
  static constexpr int kCols = SG * 16;
  static constexpr int kChunks = SG * 2;
  static constexpr int kLoadRows = 256 / kChunks;
  static constexpr int kUnits = 64 / kLoadRows;
  static constexpr int kWaveGroups = SG / 4;
};
// The plain kernel: 16-group slabs, one tile in flight (measured on MI355X
// against 8-group slabs with two 16 KiB tiles in flight: 2647 against 2659 us
// per 16-chunk call alone, 6.16-6.17 against 6.21-6.25 ms per benchmark
// step; two 32 KiB tiles in flight need more than 128 VGPRs).  The W4A4
// kernel keeps 8-group slabs: its two LDS tile buffers and four workgroups
// per CU would not fit in LDS with 16.
constexpr int kPlainSG = 16;
constexpr int kFqSG = 8;
constexpr int kTile = 64;                 // tokens per LDS tile
constexpr int kThreads = 256;
constexpr int kTargetWgs = 512;           // two workgroups on each of 256 CUs (measured best)
constexpr int kTargetWgsFq = 1024;        // fake-quant variant: ALU-heavier, four per CU hide more latency

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

__host__ __device__ inline int64_t cdiv(int64_t n, int64_t d) { return (n + d - 1) / d; }

// Work split: `total` = slabs * tiles tiles in slab-major order; workgroup w
// owns [w*total/wgs, (w+1)*total/wgs) and writes partial slot (w, s - first
// slab of w) for every slab s it touches (segs slots per workgroup).
// wgs = slabs * streams with streams = kTargetWgs / slabs, so each slab's
// token range is cut into `streams` equal parts.  Measured on MI355X: about
// two workgroups per CU, evenly spread, streams fastest (shapes that leave
// some CUs with a third workgroup run 15-20% slower).
struct Plan {
  int64_t slabs, tiles, total, wgs, segs, streams, sg;
};

Plan plan(int64_t tokens, int64_t k, int64_t target, int sg) {
  Plan p;
  p.sg = sg;
  p.slabs = cdiv(k / 16, sg);
  p.tiles = cdiv(tokens, kTile);
  p.total = p.slabs * p.tiles;
  p.streams = p.slabs < target ? target / p.slabs : 1;
  p.wgs = p.slabs < target ? p.slabs * p.streams : target;
  if (p.wgs > p.total) p.wgs = p.total;
  p.segs = p.wgs > 0 ? cdiv(cdiv(p.total, p.wgs), p.tiles) + 1 : 0;
  return p;
}

// chunk position of 16-byte chunk j of tile row R
__device__ __forceinline__ int swz(int j, int R) { return j ^ ((R >> 2) & 6); }

__device__ __forceinline__ u16x2 abs_max2(u16x2 m, uint32_t v) {
  return __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, v) & u16x2{0x7FFF, 0x7FFF});
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Quantizer state of the fake-quant variant: the code tables for the
// activations' tensor scale, built once per workgroup in LDS.
struct FqState {
  const CodeTables* t;
  const int32_t* tp;
  float s2, inv;
  bool est;     // inv = RN_f32(1 / (6 scale_2)) is finite and nonzero: arithmetic code estimate
};

// max over lanes l and l^1, which hold the two halves of one 16-element block
__device__ __forceinline__ uint32_t pair_max(uint32_t p) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)p, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  return max(p, o);
}

// Fake quantization of the lane's four 8-value chunks of a tile, in place:
// the dynamic quantizer's block code from the block max, E2M1 at that code,
// then the two-level dequantization back to bf16 (RN_f32(e2m1 * d), then
// RN_bf16).  QM is the E2M1 mode of the code tables (0 or 1: one certified
// level for every code; 2: a level per code).  The chunks pass through each
// phase together so that their table reads overlap.  amx collects the raw
// block maxima (the fused amax of the unquantized input).
template <int QM>
__device__ __forceinline__ void fake_quant_tile(uint4* v, const FqState& q, u16x2& amx) {
  static_assert(Slab<kFqSG>::kUnits == 4, "four 8-value chunks per lane and tile");
  uint32_t P[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const u16x2 m2 = abs_max2(abs_max2(abs_max2(abs_max2(u16x2{0, 0}, v[u].x), v[u].y), v[u].z), v[u].w);
    P[u] = pair_max(max((uint32_t)m2.x, (uint32_t)m2.y));
    amx = __builtin_elementwise_max(amx, u16x2{(uint16_t)P[u], 0});
  }
  int c[4];
  if (q.est) {
#pragma unroll
    for (int u = 0; u < 4; ++u) c[u] = block_code_est(P[u], q.tp, q.inv);
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) c[u] = block_code(P[u], q.tp, q.s2);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t wv[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
    float xv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) { xv[2 * i] = bf16lo(wv[i]); xv[2 * i + 1] = bf16hi(wv[i]); }
    uint32_t nb;
    if constexpr (QM == 2) nb = nibbles8(xv, c[u], *q.t, 2);
    else nb = nibbles8_level<QM>(xv, c[u], *q.t);
    const float d = q.t->d[c[u]];
    float a0, b0, a1, b1, a2, b2, a3, b3;
    fp4x2_to_f32<0>(nb, a0, b0);
    fp4x2_to_f32<1>(nb, a1, b1);
    fp4x2_to_f32<2>(nb, a2, b2);
    fp4x2_to_f32<3>(nb, a3, b3);
    const f32x2 y0 = {a0 * d, b0 * d}, y1 = {a1 * d, b1 * d}, y2 = {a2 * d, b2 * d}, y3 = {a3 * d, b3 * d};
    v[u] = make_uint4(__builtin_bit_cast(uint32_t, __builtin_convertvector(y0, bf16x2)),
                      __builtin_bit_cast(uint32_t, __builtin_convertvector(y1, bf16x2)),
                      __builtin_bit_cast(uint32_t, __builtin_convertvector(y2, bf16x2)),
                      __builtin_bit_cast(uint32_t, __builtin_convertvector(y3, bf16x2)));
  }
}

// LDS tile buffers and register tiles in flight: 1 for the plain kernel, 2
// for the fake-quant kernel.
template <int QM>
constexpr int kTileBufs = QM >= 0 ? 2 : 1;

// One workgroup's share of the partial products.  QM < 0: H += X^T X (the
// running max |x| is taken from the MFMA operands when want_amax).  QM >= 0
// (W4A4 calibration): H += Xh^T Xh with Xh = DQ(Q(X)) at the activations'
// tensor scale, quantized in registers between the load and the LDS store,
// E2M1 mode QM.  Returns the lane's packed running max |x|.
template <int QM, int SG>
__device__ __forceinline__ u16x2 partial_body(const uint16_t* __restrict__ x, int64_t tokens, int64_t k, int64_t ldx,
                                              int64_t tiles, int64_t total, int64_t wgs, int64_t segs, int64_t slabs,
                                              int64_t streams, float* __restrict__ ws, bool want_amax,
                                              uint16_t* lds_tiles, const FqState& fq) {
  using L = Slab<SG>;
  constexpr int NF = kTileBufs<QM>;                    // register tiles in flight
  int tb = 0;                                          // tiles consumed (LDS buffer parity)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t groups = k >> 4;
  // dispatch order: consecutive workgroups take neighbouring slabs of one
  // token stream (when the grid is exactly slabs x streams)
  const int64_t b = blockIdx.x;
  const int64_t w = (wgs == slabs * streams) ? (b % slabs) * streams + b / slabs : b;
  const int64_t f0 = w * total / wgs;
  const int64_t f1 = (w + 1) * total / wgs;
  const int64_t first_slab = f0 / tiles;

  // loader: thread owns chunk j = tid % kChunks of rows tid / kChunks + kLoadRows * u
  const int lj = tid & (L::kChunks - 1);
  const int lr = tid / L::kChunks;

  // MFMA reader: this wave owns groups kWaveGroups * wave + 0, 1, ... of the slab
  const int q = lane >> 4;
  const int ch = lane & 15;

  u16x2 amx = u16x2{0, 0};

  for (int64_t f = f0; f < f1;) {
    const int64_t slab = f / tiles;
    const int64_t t0 = f - slab * tiles;
    const int64_t t1 = (f1 - slab * tiles) < tiles ? (f1 - slab * tiles) : tiles;
    const int ntiles = (int)(t1 - t0);
    const int64_t gcol = slab * L::kCols + lj * 8;
    const bool col_ok = gcol < k;          // k % 16 == 0, so a chunk is all-in or all-out

    floatx4 acc[L::kWaveGroups];
#pragma unroll
    for (int i = 0; i < L::kWaveGroups; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};

    // NF tiles in flight per thread: tile i + NF is requested as soon as tile
    // i sits in LDS
    uint4 bufs[NF][L::kUnits];
    // per-lane part of the address; the tile's row offset is wave-uniform
    const int64_t lane_off = (int64_t)lr * ldx + gcol;
    auto load_tile = [&](uint4* buf, int i) {
      const int64_t r0 = (t0 + i) * kTile;
      const int64_t rows_left = tokens - r0;           // rows lr + 16u < rows_left exist
      const uint16_t* base = x + r0 * ldx;
#pragma unroll
      for (int u = 0; u < L::kUnits; ++u) {
        if (col_ok && lr + L::kLoadRows * u < rows_left) {
          // X is read exactly once: a non-temporal load keeps it from
          // displacing cached data (measured 10% faster than a plain load)
          buf[u] = ld_nt4(base + lane_off + (int64_t)(L::kLoadRows * u) * ldx);
        } else {
          buf[u] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
    };
    auto consume = [&](uint4* buf, int i) {
      if constexpr (QM >= 0) fake_quant_tile<QM>(buf, fq, amx);
      // one LDS tile: wait until every wave has read the previous one; two
      // (fake-quant kernel, measured 2-6% faster there): the barrier after
      // this write also retires the reads of the buffer written next
      if constexpr (kTileBufs<QM> == 1) __syncthreads();
      uint16_t* tile = lds_tiles + (tb % kTileBufs<QM>) * (kTile * L::kCols);
      ++tb;
#pragma unroll
      for (int u = 0; u < L::kUnits; ++u) {
        const int R = lr + L::kLoadRows * u;
        *reinterpret_cast<uint4*>(&tile[R * L::kCols + swz(lj, R) * 8]) = buf[u];
      }
      __syncthreads();
      if (i + NF < ntiles) load_tile(buf, i + NF);
#pragma unroll
      for (int gsub = 0; gsub < L::kWaveGroups; ++gsub) {
        const int gl = L::kWaveGroups * wave + gsub;   // group within the slab
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          // Two transposing reads: lane jj of each 16-lane group fetches 4
          // channels (4*(jj&3)..+3 of the group) of token R0 + jj/4, and after
          // the transpose lane ch holds its channel at 4 consecutive tokens:
          // rows 32m + 8q .. +7 of column 16 gl + ch, in order.  (Against eight 2-byte
          // reads: 5-10% faster in the fake-quant kernel; in the plain kernel
          // equal alone and 0.8% faster per benchmark step beside the sweeps,
          // from fewer instructions per tile.)
          const int jj = lane & 15;
          const int c4 = gl * 16 + 4 * (jj & 3);
          const int R0 = 32 * m + 8 * q + (jj >> 2);
          const s16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)&tile[R0 * L::kCols + swz(c4 >> 3, R0) * 8 + (c4 & 7)]);
          const s16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)&tile[(R0 + 4) * L::kCols + swz(c4 >> 3, R0 + 4) * 8 +
                                                              (c4 & 7)]);
          const u16x8 v = __builtin_bit_cast(u16x8, __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7));
          if (QM < 0 && want_amax) {
            const u32x4 d = __builtin_bit_cast(u32x4, v);
            amx = abs_max2(abs_max2(abs_max2(abs_max2(amx, d.x), d.y), d.z), d.w);
          }
          const bf16x8 a = __builtin_bit_cast(bf16x8, v);
          acc[gsub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, acc[gsub], 0, 0, 0);
        }
      }
    };

#pragma unroll
    for (int j = 0; j < NF; ++j)
      if (j < ntiles) load_tile(bufs[j], j);
    for (int i = 0; i < ntiles; i += NF) {
#pragma unroll
      for (int j = 0; j < NF; ++j)
        if (i + j < ntiles) consume(bufs[j], i + j);
    }

    // partial slot (w, slab - first_slab); lane holds C[4q + r][ch]
    float* slot = ws + ((w * segs + (slab - first_slab)) * SG) * 256;
#pragma unroll
    for (int gsub = 0; gsub < L::kWaveGroups; ++gsub) {
      const int gl = L::kWaveGroups * wave + gsub;
      if (slab * SG + gl < groups) {
#pragma unroll
        for (int r = 0; r < 4; ++r) slot[gl * 256 + (4 * q + r) * 16 + ch] = acc[gsub][r];
      }
    }
    f = slab * tiles + t1;
  }

  return amx;
}

// atomic max of the workgroup's running max |x| into *amax (as fp32 bits)
__device__ __forceinline__ void reduce_amax(u16x2 amx, float* amax) {
  __shared__ uint32_t part[kThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t am = max((uint32_t)amx.x, (uint32_t)amx.y);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) am = max(am, (uint32_t)__shfl_xor((int)am, o));
  if (lane == 0) part[wave] = am;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int i = 0; i < kThreads / 64; ++i) r = max(r, part[i]);
    if (r) atomicMax(reinterpret_cast<uint32_t*>(amax), r << 16);
  }
}

// At most 128 VGPRs (it takes 104): two of its workgroups stay resident
// beside a 256-VGPR sweep wave on every SIMD.
__global__ __launch_bounds__(kThreads, 4) void hessian_partial_kernel(const uint16_t* __restrict__ x, int64_t tokens,
                                                                       int64_t k, int64_t ldx, int64_t tiles,
                                                                       int64_t total, int64_t wgs, int64_t segs,
                                                                       int64_t slabs, int64_t streams,
                                                                       float* __restrict__ ws, float* amax) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kTile * Slab<kPlainSG>::kCols];
  // Beside a VALU-bound kernel on another stream (a sweep) this kernel's
  // waves win instruction arbitration: the memory stream is what bounds it,
  // and a pure-FMA kernel at one wave per SIMD slowed it by half at the
  // default priority, by 2% at this one.  Alone it changes nothing.
  __builtin_amdgcn_s_setprio(3);
  const FqState q{};
  const u16x2 amx = partial_body<-1, kPlainSG>(x, tokens, k, ldx, tiles, total, wgs, segs, slabs, streams, ws,
                                               amax != nullptr, tile, q);
  if (amax) reduce_amax(amx, amax);
}

// The fake-quant variant: tables first, then one loop per E2M1 mode (the
// mode is uniform over the launch, so only one loop's code runs).
__global__ __launch_bounds__(kThreads, 4) void hessian_fq_partial_kernel(const uint16_t* __restrict__ x,
                                                                          int64_t tokens, int64_t k, int64_t ldx,
                                                                          int64_t tiles, int64_t total, int64_t wgs,
                                                                          int64_t segs, int64_t slabs, int64_t streams,
                                                                          float* __restrict__ ws, float* amax,
                                                                          const float* __restrict__ scale2,
                                                                          int force_exact) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[2 * kTile * Slab<kFqSG>::kCols];
  __shared__ CodeTables t;
  __shared__ int32_t tp[128];
  FqState q;
  q.t = &t;
  q.tp = tp;
  q.s2 = *scale2;
  q.inv = (float)(1.0 / (6.0 * (double)q.s2));
  q.est = q.inv > 0.0f && q.inv < __builtin_inff();
  build_all_tables(tp, t, q.s2, force_exact);                 // syncs
  const int mode = table_mode(t);
  u16x2 amx;
  if (mode == 0)
    amx = partial_body<0, kFqSG>(x, tokens, k, ldx, tiles, total, wgs, segs, slabs, streams, ws, false, tile, q);
  else if (mode == 1)
    amx = partial_body<1, kFqSG>(x, tokens, k, ldx, tiles, total, wgs, segs, slabs, streams, ws, false, tile, q);
  else
    amx = partial_body<2, kFqSG>(x, tokens, k, ldx, tiles, total, wgs, segs, slabs, streams, ws, false, tile, q);
  if (amax) reduce_amax(amx, amax);
}

// H[g] += sum of the partials of group g over the workgroups whose range
// touches g's slab (with nchunks slot sets, those of every chunk), in fp64
// and in a fixed order (deterministic).  One workgroup per group: the
// (chunk, owner) items are cut into four contiguous ranges, one per wave,
// each lane summing float4 e of the group over its wave's range (16 loads in
// flight); wave 0 then adds H and the four sums in wave order.  (One wave per
// group had left a 16-chunk call's reduce latency-bound: 55 us at
// K = 12288.)
template <int SG>
__global__ __launch_bounds__(256) void hessian_reduce_kernel(const float4* __restrict__ ws, int64_t tiles,
                                                              int64_t total, int64_t wgs, int64_t segs, int64_t groups,
                                                              int nchunks, float4* __restrict__ H) {
  __shared__ double part[3][4][64];                           // the sums of waves 1..3
  const int64_t g = blockIdx.x;
  const int64_t s = g / SG;
  const int gl = (int)(g % SG);
  const int wave = threadIdx.x >> 6;
  const int e = threadIdx.x & 63;
  float4 h = make_float4(0.f, 0.f, 0.f, 0.f);
  if (wave == 0) h = H[g * 64 + e];
  // owning workgroups of slab s: w_lo .. w_hi (all with non-empty ranges);
  // only w_lo's range can start before slab s, so only its slot for s can
  // sit past segment 0
  const int64_t w_lo = cdiv((s * tiles + 1) * wgs, total) - 1;
  const int64_t w_hi = cdiv((s + 1) * tiles * wgs, total) - 1;
  const int n = (int)(w_hi - w_lo + 1);
  const int seg_lo = (int)(s - (w_lo * total / wgs) / tiles);
  const int sg = (int)segs;
  const int64_t chunk4 = wgs * segs * SG * 64;                // float4 per chunk's slot set
  const float4* p0 = ws + ((w_lo * segs + seg_lo) * SG + gl) * 64 + e;
  // items it = c * n + i (owner i of chunk c), chunk by chunk, then
  // workgroup order; this wave's are [it0, it1) (at most 64 * 512 items)
  const int items = nchunks * n;
  const int it0 = items * wave / 4, it1 = items * (wave + 1) / 4;
  int c = it0 / n, i = it0 - c * n;
  auto next = [&]() -> const float4* {
    const float4* q = p0 + c * chunk4 + (int64_t)(i * sg - (i ? seg_lo : 0)) * (SG * 64);
    if (++i == n) { i = 0; ++c; }
    return q;
  };
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
  int it = it0;
  for (; it + 16 <= it1; it += 16) {
    float4 v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = *next();
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      s0 += (double)v[j].x;
      s1 += (double)v[j].y;
      s2 += (double)v[j].z;
      s3 += (double)v[j].w;
    }
  }
  for (; it < it1; ++it) {
    const float4 v = *next();
    s0 += (double)v.x;
    s1 += (double)v.y;
    s2 += (double)v.z;
    s3 += (double)v.w;
  }
  if (wave > 0) {
    part[wave - 1][0][e] = s0;
    part[wave - 1][1][e] = s1;
    part[wave - 1][2][e] = s2;
    part[wave - 1][3][e] = s3;
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      s0 += part[w][0][e];
      s1 += part[w][1][e];
      s2 += part[w][2][e];
      s3 += part[w][3][e];
    }
    h.x = (float)((double)h.x + s0);
    h.y = (float)((double)h.y + s1);
    h.z = (float)((double)h.z + s2);
    h.w = (float)((double)h.w + s3);
    H[g * 64 + e] = h;
  }
}

}  // namespace

static size_t plan_bytes(const Plan& p) { return (size_t)(p.wgs * p.segs * p.sg) * 256u * sizeof(float); }

// one query for both variants: the larger of their partial buffers
size_t hessian_workspace_bytes(int64_t tokens, int64_t k) {
  const size_t a = plan_bytes(plan(tokens, k, kTargetWgs, kPlainSG));
  const size_t b = plan_bytes(plan(tokens, k, kTargetWgsFq, kFqSG));
  return a > b ? a : b;
}

template <int SG>
static int launch_reduce(const Plan& p, int64_t k, const float* ws, float* H, hipStream_t s, int nchunks = 1) {
  const int64_t groups = k / 16;
  hessian_reduce_kernel<SG><<<(unsigned)groups, 256, 0, s>>>(reinterpret_cast<const float4*>(ws), p.tiles, p.total,
                                                             p.wgs, p.segs, groups, nchunks,
                                                             reinterpret_cast<float4*>(H));
  return launch_status("hessian_reduce_kernel");
}

int launch_hessian_accum_chunks(const uint16_t* const* xs, int nchunks, int64_t tokens, int64_t k, int64_t ldx,
                                float* H, float* amax, void* workspace, hipStream_t s) {
  const Plan p = plan(tokens, k, kTargetWgs, kPlainSG);
  if (p.wgs == 0 || nchunks == 0) return NVFP4_OK;
  // One accumulate launch per chunk, each into its own partial slot set
  // (chunk c's at ws + c * chunk_floats), then one fp64 reduce over all.
  float* ws = static_cast<float*>(workspace);
  const int64_t chunk_floats = p.wgs * p.segs * kPlainSG * 256;
  for (int c = 0; c < nchunks; ++c) {
    hessian_partial_kernel<<<(unsigned)p.wgs, kThreads, 0, s>>>(xs[c], tokens, k, ldx, p.tiles, p.total, p.wgs,
                                                                 p.segs, p.slabs, p.streams, ws + c * chunk_floats,
                                                                 amax);
    const int st = launch_status("hessian_partial_kernel");
    if (st) return st;
  }
  return launch_reduce<kPlainSG>(p, k, ws, H, s, nchunks);
}

int launch_hessian_accum(const uint16_t* x, int64_t tokens, int64_t k, int64_t ldx, float* H, float* amax,
                         void* workspace, hipStream_t s) {
  return launch_hessian_accum_chunks(&x, 1, tokens, k, ldx, H, amax, workspace, s);
}

// one query for both chunk-list calls: the larger of the two per-chunk slot
// sets, times the chunk count
size_t hessian_chunks_workspace_bytes(int64_t tokens, int64_t k, int nchunks) {
  return hessian_workspace_bytes(tokens, k) * (size_t)nchunks;
}

size_t hessian_plain_workspace_bytes(int64_t tokens, int64_t k) {
  return plan_bytes(plan(tokens, k, kTargetWgs, kPlainSG));
}

// Device address of `scratch` per device, looked up once per device with
// that device current (each device holds its own copy of the array).
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64] = {};

static int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return NVFP4_ERR_BAD_INPUT;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return hip_status(hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return NVFP4_OK;
}

// The plain accumulate with its partial slots in `scratch` (the caller has
// checked that the plan fits).  Every slot the reduce reads is written by
// the partial kernel of the same call, so nothing needs clearing.
int launch_hessian_accum_noalloc(const uint16_t* x, int64_t tokens, int64_t k, int64_t ldx, float* H, float* amax,
                                 hipStream_t s) {
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st) return st;
  return launch_hessian_accum(x, tokens, k, ldx, H, amax, ws, s);
}

int launch_hessian_accum_fq_chunks(const uint16_t* const* xs, int nchunks, int64_t tokens, int64_t k, int64_t ldx,
                                   const float* scale2, float* H, float* amax, void* workspace, hipStream_t s) {
  const Plan p = plan(tokens, k, kTargetWgsFq, kFqSG);
  if (p.wgs == 0 || nchunks == 0) return NVFP4_OK;
  // as the plain chunk list: one accumulate launch per chunk into its own
  // partial slot set, one fp64 reduce over all of them
  float* ws = static_cast<float*>(workspace);
  const int64_t chunk_floats = p.wgs * p.segs * kFqSG * 256;
  const int fx = force_exact_flag();
  for (int c = 0; c < nchunks; ++c) {
    hessian_fq_partial_kernel<<<(unsigned)p.wgs, kThreads, 0, s>>>(xs[c], tokens, k, ldx, p.tiles, p.total, p.wgs,
                                                                    p.segs, p.slabs, p.streams, ws + c * chunk_floats,
                                                                    amax, scale2, fx);
    const int st = launch_status("hessian_fq_partial_kernel");
    if (st) return st;
  }
  return launch_reduce<kFqSG>(p, k, ws, H, s, nchunks);
}

int launch_hessian_accum_fq(const uint16_t* x, int64_t tokens, int64_t k, int64_t ldx, const float* scale2, float* H,
                            float* amax, void* workspace, hipStream_t s) {
  return launch_hessian_accum_fq_chunks(&x, 1, tokens, k, ldx, scale2, H, amax, workspace, s);
}

}  // namespace nvfp4
