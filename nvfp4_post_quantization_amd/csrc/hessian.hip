// Block-diagonal local Hessian accumulation ("Coder390 NVFP4 校正（校准）方式"
// §2 step 2):  H[g] += X_g^T X_g  for every group g of 16 input channels.
//
// The work is HBM-bound (2 bytes read per element, 32 flops per element), so
// the design goal is a single coalesced pass over X:
//  * a workgroup owns a slab of 8 groups (128 channels, 256 B of every token
//    row) and a contiguous token range; 64-token tiles are staged through LDS
//    (16 B per lane, coalesced rows);
//  * H_g = X_g^T X_g is a 16x16 contraction over tokens, done with
//    v_mfma_f32_16x16x32_bf16.  In that instruction lane l supplies row l%16
//    of A and column l%16 of B for K-slots 8*(l/16)..+7; for A = X_g^T and
//    B = X_g both are "channel l%16 at 8 tokens", so one register feeds both
//    operands.  The lane reads its 8 tokens of one channel from LDS; the
//    16-byte chunks are XOR-swizzled by row so the four lane groups of a read
//    hit disjoint banks;
//  * each workgroup writes its fp32 partial H to the workspace; a second
//    kernel adds the partials to H in fp64, in split order (deterministic).
// Optionally the running max |x| (calibration step 1) is taken from the same
// loads.
#include "common.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

constexpr int kSlabGroups = 8;            // groups per workgroup
constexpr int kSlabCols = kSlabGroups * 16;
constexpr int kTile = 64;                 // tokens per LDS tile
constexpr int kRowBytes = kSlabCols * 2;  // 256
constexpr int kThreads = 256;
constexpr int kTargetWgs = 2048;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

struct Split {
  int64_t slabs, splits, tiles_per_split;
};

Split plan(int64_t tokens, int64_t k) {
  Split p;
  int64_t groups = k / 16;
  p.slabs = (groups + kSlabGroups - 1) / kSlabGroups;
  int64_t tiles = (tokens + kTile - 1) / kTile;
  int64_t want = (kTargetWgs + p.slabs - 1) / p.slabs;
  if (want < 1) want = 1;
  if (want > tiles) want = tiles;
  p.tiles_per_split = (tiles + want - 1) / want;
  p.splits = (tiles + p.tiles_per_split - 1) / p.tiles_per_split;
  return p;
}

// chunk position of 16-byte chunk j of tile row R
__device__ __forceinline__ int swz(int j, int R) { return j ^ ((R >> 2) & 6); }

__global__ __launch_bounds__(kThreads) void hessian_partial_kernel(const uint16_t* __restrict__ x, int64_t tokens,
                                                                    int64_t k, int64_t ldx, int64_t tiles_per_split,
                                                                    float* __restrict__ ws, float* amax) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kTile * kSlabCols];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t groups = k >> 4;
  const int64_t slab = blockIdx.x;
  const int64_t split = blockIdx.y;
  const int64_t col0 = slab * kSlabCols;
  const int64_t t_begin = split * tiles_per_split * kTile;
  int64_t t_end = t_begin + tiles_per_split * kTile;
  if (t_end > tokens) t_end = tokens;
  const int ntiles = (int)((t_end - t_begin + kTile - 1) / kTile);

  // loader: thread owns chunk j = tid%16 of rows tid/16 + 16*i
  const int lj = tid & 15;
  const int lr = tid >> 4;
  const int64_t gcol = col0 + lj * 8;
  const bool col_ok = gcol < k;            // k % 16 == 0, so a chunk is all-in or all-out

  // MFMA reader: this wave owns groups 2*wave and 2*wave+1 of the slab
  const int q = lane >> 4;
  const int ch = lane & 15;

  floatx4 acc[2];
  acc[0] = floatx4{0.f, 0.f, 0.f, 0.f};
  acc[1] = floatx4{0.f, 0.f, 0.f, 0.f};
  uint32_t amx = 0;

  uint4 buf[4];
  auto load_tile = [&](int tt) {
    const int64_t r0 = t_begin + (int64_t)tt * kTile;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = r0 + lr + 16 * i;
      if (col_ok && row < t_end) {
        buf[i] = *reinterpret_cast<const uint4*>(x + row * ldx + gcol);
      } else {
        buf[i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };

  if (ntiles > 0) load_tile(0);
  for (int tt = 0; tt < ntiles; ++tt) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int R = lr + 16 * i;
      *reinterpret_cast<uint4*>(&tile[R * kSlabCols + swz(lj, R) * 8]) = buf[i];
      if (amax) {
        uint32_t v[4] = {buf[i].x, buf[i].y, buf[i].z, buf[i].w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          amx = max(amx, v[w] & 0x7FFFu);
          amx = max(amx, (v[w] >> 16) & 0x7FFFu);
        }
      }
    }
    __syncthreads();
    if (tt + 1 < ntiles) load_tile(tt + 1);
#pragma unroll
    for (int gsub = 0; gsub < 2; ++gsub) {
      const int gl = 2 * wave + gsub;                 // group within the slab
      const int col = gl * 16 + ch;                   // column within the slab
      const int j = col >> 3, within = col & 7;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        u16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int R = 32 * m + 8 * q + e;
          v[e] = tile[R * kSlabCols + swz(j, R) * 8 + within];
        }
        bf16x8 a = __builtin_bit_cast(bf16x8, v);
        acc[gsub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, acc[gsub], 0, 0, 0);
      }
    }
  }

  // partial H: lane holds C[4q + r][ch]
#pragma unroll
  for (int gsub = 0; gsub < 2; ++gsub) {
    const int64_t g = slab * kSlabGroups + 2 * wave + gsub;
    if (g < groups) {
      float* dst = ws + (split * groups + g) * 256;
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(4 * q + r) * 16 + ch] = acc[gsub][r];
    }
  }
  if (amax) {
    __shared__ uint32_t part[kThreads / 64];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amx = max(amx, (uint32_t)__shfl_xor((int)amx, o));
    if (lane == 0) part[wave] = amx;
    __syncthreads();
    if (tid == 0) {
      uint32_t r = 0;
      for (int i = 0; i < kThreads / 64; ++i) r = max(r, part[i]);
      if (r) atomicMax(reinterpret_cast<uint32_t*>(amax), r << 16);
    }
  }
}

// H[e] += sum over splits of ws[split][e], in fp64, split order fixed.
__global__ __launch_bounds__(256) void hessian_reduce_kernel(const float* __restrict__ ws, int64_t splits,
                                                              int64_t n, float* __restrict__ H) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  double s = 0.0;
  for (int64_t p = 0; p < splits; ++p) s += (double)ws[p * n + i];
  H[i] = (float)((double)H[i] + s);
}

}  // namespace

size_t hessian_workspace_bytes(int64_t tokens, int64_t k) {
  Split p = plan(tokens, k);
  return (size_t)p.splits * (size_t)(k / 16) * 256u * sizeof(float);
}

int launch_hessian_accum(const uint16_t* x, int64_t tokens, int64_t k, int64_t ldx, float* H, float* amax,
                         void* workspace, hipStream_t s) {
  Split p = plan(tokens, k);
  float* ws = static_cast<float*>(workspace);
  dim3 grid((unsigned)p.slabs, (unsigned)p.splits, 1);
  hessian_partial_kernel<<<grid, kThreads, 0, s>>>(x, tokens, k, ldx, p.tiles_per_split, ws, amax);
  int st = launch_status("hessian_partial_kernel");
  if (st) return st;
  const int64_t n = (k / 16) * 256;
  hessian_reduce_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(ws, p.splits, n, H);
  return launch_status("hessian_reduce_kernel");
}

}  // namespace nvfp4
