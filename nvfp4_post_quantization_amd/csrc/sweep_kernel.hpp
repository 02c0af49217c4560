// Device code of the Hessian-weighted block-scale sweep, shared by the two
// translation units that instantiate it: sweep.hip (sweep_kernel<false>, the
// kernel of nvfp4_scale_sweep) and sweep_stats.hip (sweep_kernel<true>, its
// counting build for nvfp4_scale_sweep_stats).  Each unit instantiates one
// kernel only: with both in one unit the compiler stopped inlining the
// per-group set-up into the plain kernel, which then spilled registers.
//
// The sweep (fp8_scale_sweep, "Coder390 NVFP4
// 校正（校准）方式" §2 step 3): for each 16-element weight block w of group g
// and each finite code c, cost(c) = e^T H_g e with e = w - q(c) d_c; keep the
// code of least cost (lowest code on ties).
//
// Search order and exact pruning
// ------------------------------
// Evaluating all 127 codes per block is wasted work: far from the block's
// max-based code the cost is provably large.  For symmetric positive
// semidefinite H and any element i,
//     e^T H e >= S_i e_i^2,   S_i = 1 / (H^-1)_ii   (Schur complement of H).
// At a code c every element with |w_i| > 6 d_c saturates, and for all codes
// c' <= c:  |e_i| >= |w_i| - 6 d_c.  At a code c every element with
// |w_i| <= d_c / 4 quantizes to zero, and for all codes c' >= c: e_i = w_i.
// Both bounds are monotone, so one check disposes of a whole side:
//     LB_low(c)  = max_i S_i (|w_i| - 6 d_c)_+^2       (all codes <= c)
//     LB_high(c) = max_{i : |w_i| <= d_c/4} S_i w_i^2   (all codes >= c)
// Where the diagonal screen below is on (Gershgorin row sums r_i <= 0.9 in
// H_g's unit-diagonal scaling), the same per-element errors also give sum
// bounds, e^T H e >= (1 - max r) sum_i H_ii e_i^2:
//     LB'_low(c)  = (1 - max r) sum_i H_ii (|w_i| - 6 d_c)_+^2
//     LB'_high(c) = (1 - max r) sum_{i : |w_i| <= d_c/4} H_ii w_i^2
// and there a side closes on the sum bound alone (otherwise on the max
// bound).  With several saturating or vanishing elements the sum bound is the
// larger one, and it ends the long searches that decide a wave's time
// (measured on MI355X against the max bounds: 15.7 -> 14.9 codes per block on
// the MLP weights, the three sweeps 2.40 -> 2.22 ms, the q_proj sweep 159 ->
// 99 us; keeping the max bounds beside the sum bounds evaluated 0.05% fewer
// codes and was 2.5% slower; outputs bit for bit unchanged).
// Each block evaluates code 0 and its max-based code c0, then grows a window
// [lo, hi] around c0 by one code per step, alternating sides, and closes a
// side once its bound exceeds the best cost found by a margin (2e-5
// relative) that covers every fp32/fp64 rounding involved, so every pruned
// code is strictly worse than the answer.  S_i come from an fp64 Cholesky of
// H_g and are scaled down by 1e-5; a group whose H_g is not safely positive
// definite gets S = 0, so its bounds prune nothing while the best cost is
// positive.  A best cost of exactly 0 ends a block's search (no code costs
// less), and a negative one (fp32 rounding of a form whose true value is
// about zero, on a singular H) closes both sides at once, since the closing
// test compares a square with a negative threshold: every code's true cost
// is at least 0, within rounding of the one kept.
//
// Mapping on gfx950
// -----------------
//  * a workgroup = 4 waves = 4 adjacent groups; lane l of wave w handles rows
//    r0 + l (+64, ...) of group 4*blockIdx.x + w, so the four waves read each
//    row's 128 contiguous bytes together, and H_g is uniform per wave (staged
//    in LDS once; the compiler keeps its upper triangle in VGPRs for the
//    step loop);
//  * per step every lane evaluates one code of its own block: E2M1
//    quantization by the certified FP4-convert paths (nvfp4_device.hpp), then
//    the symmetric quadratic form 2 * sum_i e_i (H_ii e_i / 2 + sum_{j>i}
//    H_ij e_j) in fp32 (152 VALU ops); the table values of the two candidate
//    codes are held in registers and fetched one step ahead;
//  * a diagonal screen comes first: when H_g's unit-diagonal scaling has
//    Gershgorin row sums r_i <= 0.9, e^T H e >= (1 - max r) sum_i H_ii e_i^2,
//    and a wave whose searching lanes all have that bound above the
//    threshold skips the form for this step (on the MLP calibration
//    workload about half the steps; 32 extra ops per step).  Codes it skips
//    could not have won, so the outputs are those of the unscreened search,
//    bit for bit;
//  * the wave steps until all its lanes are done (lanes that finish early
//    idle); the nibbles are re-quantized at the chosen code.
//  * weights are read with non-temporal loads, workgroups are ordered so
//    that 32 x-neighbours share an XCD, and outputs go through LDS: the last
//    of a workgroup's waves to finish writes all its rows, four groups (32
//    bytes of nibbles, 4 code bytes) per row at a time.  The sweep runs
//    beside the HBM-bound Hessian accumulate, which its row-scattered reads
//    and writes had slowed by about 8%;
//  * two workgroups per CU (launch bounds): 256 VGPRs, no scratch.  The
//    occupancy-capped launch (one workgroup per CU, for running beside
//    another kernel) reserves dynamic LDS so that a second one cannot fit.
// fp32 MFMA and fp32 VALU share one datapath on this chip (measured: their
// times add), so a dense MFMA product would not be cheaper than the
// symmetric VALU form; pruning is what removes work.
// H is taken as symmetric (its upper triangle is used), as the accumulate
// entry point produces it.
#pragma once

#include "common.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr float kPruneMargin = 2e-5f;
// Target workgroups per launch (the MLP weights, same process: 2048 against
// 4096 took the down sweep from 0.905 to 0.81 ms and the gate sweep from
// 0.873 to 0.838 ms, half the per-workgroup set-up; 512 was 3% slower), and
// the fewest rows per workgroup: two 64-row batches, so that a small weight's
// workgroups amortise their set-up (the [2048, 2048] q_proj: 157 us in 512
// workgroups of 128 rows against 162 us in 1024 of 64).
constexpr int64_t kSweepWgs = 2048;
constexpr int64_t kMinRowsPerWg = 128;
// Rows of a workgroup's outputs that can be staged in LDS (8 batches of 64);
// the launcher keeps rows_per_wg within it for any row count below 2^25.
constexpr int kStageRows = 512;
constexpr int kStageBatches = kStageRows / 64;

// Value of v in lane src (a constant), broadcast through scalar registers.
__device__ __forceinline__ double bcast(double v, int src) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, src);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), src);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// sqrt(S_i) of the wave's group, S_i = (1 - 1e-5) / (H^-1)_ii in fp64, H taken
// from its upper triangle (as the cost is); all zero when H is not safely positive definite.
// Lanes 0..15 own rows 0..15 (higher lanes duplicate them).  Writes out[0..15].
__device__ void schur_sqrt(const float* __restrict__ Hg, int lane, float* out) {
  const int i = lane & 15;
  double a[16];
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) a[kk] = (double)Hg[kk < i ? kk * 16 + i : i * 16 + kk];   // upper triangle
  bool ok = true;
  double pmax = 0.0, pmin = 1e300;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const double pj = bcast(a[j], j);               // updated A_jj from lane j
    ok = ok && (pj > 0.0);
    pmax = fmax(pmax, pj);
    pmin = fmin(pmin, pj);
    const double ljj = ok ? sqrt(pj) : 1.0;
    const double lij = a[j] / ljj;                  // L_ij (meaningful for i >= j)
    a[j] = lij;
#pragma unroll
    for (int kk = j + 1; kk < 16; ++kk) {
      const double lkj = bcast(lij, kk);
      if (i >= kk) a[kk] -= lij * lkj;
    }
  }
  // column i of L^-1 by forward substitution; (H^-1)_ii = sum_k y_k^2
  double y[16];
  double s = 0.0;
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) {
    double acc = (kk == i) ? 1.0 : 0.0;
#pragma unroll
    for (int m = 0; m < kk; ++m) acc -= bcast(a[m], kk) * y[m];
    y[kk] = acc / bcast(a[kk], kk);
    s += y[kk] * y[kk];
  }
  ok = ok && (pmin > 1e-9 * pmax) && (s > 0.0);
  const double S = ok ? (1.0 - 1e-5) / s : 0.0;
  if (lane < 16) out[lane] = (float)sqrt(S);
}

// e = w - q d for the 16 elements from their nibbles nb at block scale d.
__device__ __forceinline__ void error_from_nibbles(const float* wv, uint2 nb, float d, float* e) {
  float q[16];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t w = h ? nb.y : nb.x;
    fp4x2_to_f32<0>(w, q[8 * h + 0], q[8 * h + 1]);
    fp4x2_to_f32<1>(w, q[8 * h + 2], q[8 * h + 3]);
    fp4x2_to_f32<2>(w, q[8 * h + 4], q[8 * h + 5]);
    fp4x2_to_f32<3>(w, q[8 * h + 6], q[8 * h + 7]);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) e[i] = fmaf(-q[i], d, wv[i]);
}

// e = w - q d for the 16 elements at code c (lane-varying), exact quantization.
__device__ __forceinline__ void block_error(const float* wv, int c, const CodeTables& t, int mode, float* e) {
  error_from_nibbles(wv, nibbles16(wv, c, t, mode), t.d[c], e);
}

// e^T H e with the upper triangle of H (wave-uniform, in LDS: broadcast reads):
// 2 * sum_i e_i (hh_i e_i + sum_{j>i} H_ij e_j), hh_i = H_ii / 2.
__device__ __forceinline__ float quad_form(const float* e, const float* Hg, const float* hh) {
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float v = hh[i] * e[i];
#pragma unroll
    for (int j = i + 1; j < 16; ++j) v = fmaf(Hg[i * 16 + j], e[j], v);
    acc = fmaf(e[i], v, acc);
  }
  return 2.0f * acc;
}

// Factor of the diagonal screen for group H_g (every lane returns it; 0 =
// screen off).  With r_i = sum_{j != i} |H_ij| / sqrt(H_ii H_jj) (upper
// triangle mirrored), Gershgorin's theorem on the unit-diagonal scaling of H
// gives e^T H e >= (1 - max_i r_i) sum_i H_ii e_i^2.  The screen is used only
// when max_i r_i <= 0.9: then the fp32 quadratic form's relative rounding
// error stays below 2e-5 (its absolute terms sum to at most (1 + r)/(1 - r)
// times its value), well inside the 1e-4 margin taken here plus the pruning
// margin, so a screened-out code is one whose computed cost exceeds the best.
// Returns 2 (1 - max r)(1 - 1e-4), the factor of sum_i e_i (H_ii / 2) e_i.
__device__ float screen_factor(const float* Hg, int lane) {
  const int i = lane & 15;
  const double hii = (double)Hg[i * 17];
  double r = 0.0;
  bool ok = hii > 0.0 && hii < 1e300;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const double hjj = (double)Hg[j * 17];
    ok = ok && hjj > 0.0 && hjj < 1e300;
    const double hij = (double)Hg[j < i ? j * 16 + i : i * 16 + j];
    r += (j != i && ok) ? fabs(hij) / sqrt(hii * hjj) : 0.0;
  }
  ok = ok && r <= 0.9;                                       // false for NaN too
  double rmax = 0.0;
  bool all_ok = true;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    rmax = fmax(rmax, bcast(r, j));
    all_ok = all_ok && __builtin_amdgcn_readlane((int)ok, j) != 0;
  }
  return all_ok ? (float)(2.0 * (1.0 - rmax) * (1.0 - 1e-4)) : 0.0f;
}

// The window search of one block around its max-based code c0 (code 0 and
// c0 already evaluated into best/bestc), closing each side by its Schur
// bound.  MODE 0 and 1 (one fast level for every code): the table values of
// the two candidates, codes lo - 1 and hi + 1, stay in registers, and when a
// side advances its replacement is requested from LDS at once and taken in
// at the top of the next step, so the lookup's latency hides behind this
// step's quantization and quadratic form.  MODE 2 (per-code levels) reads
// the tables at each step.  Every lane computes exactly what the table reads
// would give.
// XCD-aware workgroup order.  The dispatcher places workgroup L (linear id)
// on XCD L % 8, and each XCD has its own L2.  Runs of kXcdBand workgroups
// that are neighbours in x (the same rows, consecutive groups: 32 x 4 groups
// = 1 KiB of each row's packed output and 128 bytes of its codes, whole
// lines) are placed on one XCD instead of spread over all eight, so that
// their reads of a row's weights and their writes of its outputs meet in one
// L2.  Measured beside the Hessian accumulate: 0.2-0.25 ms less per
// benchmark step.  A permutation of the grid; the last (total mod 8
// kXcdBand) workgroups keep their place.
constexpr uint32_t kXcds = 8;
constexpr uint32_t kXcdBand = 32;

__device__ __forceinline__ void sweep_wg_coords(int64_t* bx, int64_t* by) {
  const uint32_t gx = gridDim.x, total = gx * gridDim.y;
  const uint32_t L = blockIdx.x + blockIdx.y * gx;
  const uint32_t full = total / (kXcdBand * kXcds) * (kXcdBand * kXcds);
  uint32_t lam = L;
  if (L < full) {
    const uint32_t c = L % kXcds, s = L / kXcds;
    const uint32_t xi = s % kXcdBand, q = kXcds * (s / kXcdBand) + c;
    lam = q * kXcdBand + xi;
  }
  *bx = lam % gx;
  *by = lam / gx;
}

// Work counters of the counting build (wave-uniform, in scalar registers).
struct SweepStats {
  uint32_t evals, steps, forms, screens;
};

template <int MODE, bool STATS>
__device__ __forceinline__ void search_block(const float* wv, const float* a, const float* b, int c0, bool done,
                                             float& best, int& bestc, const CodeTables& t, const float* Hg,
                                             const float* hh, float thr_scale, float mu2, SweepStats& st) {
  // table values of code c on the mode's level: d, reciprocal (level 0: r,
  // level 1: rh) and the reciprocal's low part (level 1 only)
  auto rec = [&](int c) { return MODE == 0 ? t.r[c] : t.rh[c]; };
  auto low = [&](int c) { return MODE == 1 ? t.rl[c] : 0.0f; };
  float dl = 0.0f, ql = 0.0f, pl = 0.0f, dh = 0.0f, qh = 0.0f, ph = 0.0f;
  float nd = 0.0f, nq = 0.0f, np = 0.0f;                    // requested replacement, not yet taken in
  bool nlo = false, npend = false;
  if constexpr (MODE != 2) {                                 // 1 <= c0 <= 126
    dl = t.d[c0 - 1]; ql = rec(c0 - 1); pl = low(c0 - 1);
    dh = t.d[c0 + 1]; qh = rec(c0 + 1); ph = low(c0 + 1);
  }
  int lo = c0, hi = c0, side = 0;
  bool done_lo = false, done_hi = false;
  // Branch-free steps (selects instead of divergent ifs: the exec-mask
  // bookkeeping of nested ifs cost more issue slots than the bounds do).
  while (true) {
    if constexpr (MODE != 2) {
      const bool in_lo = npend && nlo, in_hi = npend && !nlo;
      dl = in_lo ? nd : dl; ql = in_lo ? nq : ql; pl = in_lo ? np : pl;
      dh = in_hi ? nd : dh; qh = in_hi ? nq : qh; ph = in_hi ? np : ph;
    }
    // both bounds for every lane (1 <= lo and hi <= 126, so the reads are
    // in bounds; a side already closed, or at the end of the range, ignores
    // its value)
    const float dlo = MODE == 2 ? t.d[lo - 1] : dl;
    const float dhi = MODE == 2 ? t.d[hi + 1] : dh;
    const float thr = best * thr_scale;
    const float x = 6.0f * dlo, qz = 0.25f * dhi;
    float mlo = 0.0f, mhi = 0.0f, slo = 0.0f, shi = 0.0f;
    if (mu2 > 0.0f) {                                        // wave-uniform
      // the sum bounds (the screen's condition holds for this group)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool z = fabsf(wv[i]) <= qz;
        const float el = fmaxf(fabsf(wv[i]) - x, 0.0f);
        slo = fmaf(hh[i] * el, el, slo);
        const float eh = z ? wv[i] : 0.0f;
        shi = fmaf(hh[i] * eh, eh, shi);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        mlo = fmaxf(mlo, fmaf(-x, b[i], a[i]));
        mhi = fmaxf(mhi, fabsf(wv[i]) <= qz ? a[i] : 0.0f);
      }
    }
    const bool act = !done;
    done_lo = done_lo || (act && (lo <= 1 || mlo * mlo > thr || mu2 * slo > thr));
    done_hi = done_hi || (act && (hi >= kCodes - 1 || mhi * mhi > thr || mu2 * shi > thr));
    const bool cont = act && !(done_lo && done_hi);
    done = !cont;
    const bool take_lo = cont && !done_lo && (done_hi || side == 0);
    const int next = cont ? (take_lo ? lo - 1 : hi + 1) : c0;
    side ^= cont ? 1 : 0;
    if (!__any(cont)) break;                                 // wave-uniform exit; at most 126 steps
    if constexpr (STATS) {
      st.steps += 1;
      st.evals += (uint32_t)__popcll(__ballot(cont));
    }
    float e[16];
    if constexpr (MODE == 2) {
      block_error(wv, next, t, 2, e);
    } else {
      const float d = take_lo ? dl : dh, q = take_lo ? ql : qh, p = take_lo ? pl : ph;
      // the replacement for the side that advances (1 <= next <= 126, so in bounds)
      const int nc = take_lo ? next - 1 : next + 1;
      nd = t.d[nc]; nq = rec(nc); np = low(nc);
      nlo = take_lo;
      npend = true;
      error_from_nibbles(wv, make_uint2(nibbles8_vals<MODE>(wv, d, q, p), nibbles8_vals<MODE>(wv + 8, d, q, p)),
                         d, e);
    }
    // Diagonal screen (mu2 > 0, wave-uniform): the full form is skipped when
    // no searching lane's diagonal bound mu2 * sum_i H_ii e_i^2 / 2 stays
    // within the threshold; the forms that are computed are unchanged.
    float cc;
    if (mu2 > 0.0f) {
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) s = fmaf(e[i] * e[i], hh[i], s);
      const bool need = cont && !(mu2 * s > thr);
      if constexpr (STATS) st.screens += 1;
      if (__any(need)) {
        cc = quad_form(e, Hg, hh);
        if constexpr (STATS) st.forms += 1;
      } else {
        cc = __builtin_inff();
      }
    } else {
      cc = quad_form(e, Hg, hh);
      if constexpr (STATS) st.forms += 1;
    }
    lo = (cont && take_lo) ? next : lo;
    hi = (cont && !take_lo) ? next : hi;
    const bool better = cont && (cc < best || (cc == best && next < bestc));
    best = better ? cc : best;
    bestc = better ? next : bestc;
  }
}

// STATS = true: the counting build of nvfp4_scale_sweep_stats (same search,
// same outputs), which writes no costs: its `cost` argument carries the
// uint64 counter array instead, to which each wave adds its counts.  (The
// parameter list is shared so that the plain build keeps its registers: an
// extra kernel argument made it spill.)
template <bool STATS>
__global__ __launch_bounds__(kThreads, 2) void sweep_kernel(const uint16_t* __restrict__ w, int64_t rows, int64_t k,
                                                         int64_t ldw, const float* __restrict__ H,
                                                         const float* __restrict__ scale2, int64_t rows_per_wg,
                                                         uint8_t* __restrict__ packed, uint8_t* __restrict__ codes,
                                                         float* __restrict__ cost, int force_exact) {
  __shared__ CodeTables t;
  __shared__ int32_t tp[128];
  __shared__ float sqS[kWaves][16];
  __shared__ __attribute__((aligned(16))) float Hs[kWaves][256];
  // Output staging: each wave puts its batches' nibbles and codes here, and
  // the last of the workgroup's waves to finish writes them all out, a row's
  // four groups together (one 32-byte nibble segment and one 4-byte code word
  // per row instead of four 8-byte and four 1-byte stores at different
  // times).
  __shared__ __attribute__((aligned(16))) uint2 st_nib[kStageRows][kWaves];
  __shared__ uint32_t st_code[kStageRows];
  __shared__ uint32_t st_done[kStageBatches];
  const float s2 = *scale2;
  if (threadIdx.x < kStageBatches) st_done[threadIdx.x] = 0u;
  build_all_tables(tp, t, s2, force_exact);                     // syncs
  const int mode = table_mode(t);

  const int64_t groups = k >> 4;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t bx, by;
  sweep_wg_coords(&bx, &by);
  const int64_t g0 = bx * kWaves;                            // the workgroup's first group
  const int64_t g = g0 + wave;
  if (g < groups) {
    schur_sqrt(H + g * 256, lane, sqS[wave]);
#pragma unroll
    for (int i = 0; i < 4; ++i) Hs[wave][lane + 64 * i] = H[g * 256 + lane + 64 * i];
  }
  __syncthreads();
  if (g >= groups) return;                                   // no barrier after this point

  const float* Hg = Hs[wave];
  float hh[16], b[16];                                       // wave-uniform: kept in scalar registers
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    hh[i] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(0.5f * Hg[i * 17])));
    b[i] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sqS[wave][i])));
  }
  const float thr_scale = 1.0f + kPruneMargin;
  const float mu2 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(screen_factor(Hg, lane))));

  const int64_t r0 = by * rows_per_wg;
  int64_t r1 = r0 + rows_per_wg;
  if (r1 > rows) r1 = rows;
  SweepStats st{0u, 0u, 0u, 0u};
  uint32_t n_blocks = 0;

  for (int64_t rb = r0; rb < r1; rb += 64) {
    const int64_t r = rb + lane;
    const bool valid = r < r1;
    float wv[16];
    {
      const int64_t rr = valid ? r : rb;                     // rb < r1 always holds
      const uint4* src = reinterpret_cast<const uint4*>(w + rr * ldw + g * 16);
      // non-temporal: a weight is read once (measured beside the Hessian
      // accumulate: 0.15 ms less per benchmark step than cached loads)
      const uint4 v0 = ld_nt4(src), v1 = ld_nt4(src + 1);
      const uint32_t u[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) { wv[2 * i] = bf16lo(u[i]); wv[2 * i + 1] = bf16hi(u[i]); }
    }
    float a[16];
    uint32_t P = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      a[i] = b[i] * fabsf(wv[i]);
      P = max(P, (__float_as_uint(wv[i]) >> 16) & 0x7FFFu);
    }
    // code 0 (zero scale): e = w
    float best = quad_form(wv, Hg, hh);
    int bestc = 0;
    // nothing beats cost 0 (and code 0 is the lowest); with scale_2 = 0 every code costs w^T H w
    bool done = !valid || best == 0.0f || s2 == 0.0f;
    int c0 = block_code(P, tp, s2);
    c0 = c0 < 1 ? 1 : (c0 > kCodes - 1 ? kCodes - 1 : c0);
    {
      float e[16];
      block_error(wv, c0, t, mode, e);
      const float cc = quad_form(e, Hg, hh);
      if (!done && cc < best) { best = cc; bestc = c0; }      // c0 > 0: a tie keeps code 0
    }
    if constexpr (STATS) {                                   // code 0 and c0, every lane computed
      st.steps += 2;
      st.forms += 2;
      st.evals += (uint32_t)(__popcll(__ballot(valid)) + __popcll(__ballot(!done)));
      n_blocks += (uint32_t)__popcll(__ballot(valid));
    }
    if (mode == 0) {
      search_block<0, STATS>(wv, a, b, c0, done, best, bestc, t, Hg, hh, thr_scale, mu2, st);
    } else if (mode == 1) {
      search_block<1, STATS>(wv, a, b, c0, done, best, bestc, t, Hg, hh, thr_scale, mu2, st);
    } else {
      search_block<2, STATS>(wv, a, b, c0, done, best, bestc, t, Hg, hh, thr_scale, mu2, st);
    }
    const uint2 nb = nibbles16(wv, bestc, t, mode);
    float* const cost_out = STATS ? nullptr : cost;
    if (rows_per_wg > kStageRows) {                          // (only for huge row counts) direct stores
      if (valid) {
        *reinterpret_cast<uint2*>(packed + r * (k >> 1) + g * 8) = nb;
        codes[r * groups + g] = (uint8_t)bestc;
        if (cost_out) cost_out[r * groups + g] = best;
      }
      continue;
    }
    const int j = (int)((rb - r0) >> 6);                     // batch within the workgroup
    const int sr = j * 64 + lane;                            // staging row
    st_nib[sr][wave] = nb;
    reinterpret_cast<uint8_t*>(&st_code[sr])[wave] = (uint8_t)bestc;
    if (cost_out && valid) cost_out[r * groups + g] = best;   // optional output: not staged
    // publish the batch; the wave that completes the count writes it out
    // (the release orders every lane's staging stores before lane 0's add)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    uint32_t prev = 0;
    if (lane == 0)
      prev = __hip_atomic_fetch_add(&st_done[j], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    prev = (uint32_t)__builtin_amdgcn_readlane((int)prev, 0);
    // waves of this workgroup with a group (the others returned above); each
    // wave runs the batches in order, so the last to finish the last batch
    // is the last to finish, and it writes every batch out
    const uint32_t nw = (uint32_t)(groups - g0 < kWaves ? groups - g0 : kWaves);
    const int nbat = (int)((r1 - r0 + 63) >> 6);
    if (j == nbat - 1 && prev + 1 == nw) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      // whole-row-segment stores where the destinations allow them (uniform)
      const bool nib16 = nw == kWaves && ((k >> 1) % 16) == 0 && (reinterpret_cast<uintptr_t>(packed) & 15) == 0;
      const bool code4 = nw == kWaves && (groups % 4) == 0 && (reinterpret_cast<uintptr_t>(codes) & 3) == 0;
      for (int jb = 0; jb < nbat; ++jb) {
        const int sw = jb * 64 + lane;                       // staging row of output row ro
        const int64_t ro = r0 + jb * 64 + lane;
        if (ro < r1) {
          uint8_t* pd = packed + ro * (k >> 1) + g0 * 8;
          if (nib16) {
            const uint4* src = reinterpret_cast<const uint4*>(&st_nib[sw][0]);
            reinterpret_cast<uint4*>(pd)[0] = src[0];
            reinterpret_cast<uint4*>(pd)[1] = src[1];
          } else {
            for (uint32_t q = 0; q < nw; ++q) reinterpret_cast<uint2*>(pd)[q] = st_nib[sw][q];
          }
          uint8_t* cd = codes + ro * groups + g0;
          const uint32_t cw = st_code[sw];
          if (code4) {
            *reinterpret_cast<uint32_t*>(cd) = cw;
          } else {
            for (uint32_t q = 0; q < nw; ++q) cd[q] = (uint8_t)(cw >> (8 * q));
          }
        }
      }
    }
  }
  if constexpr (STATS) {
    unsigned long long* stats = reinterpret_cast<unsigned long long*>(cost);
    if (lane == 0) {
      atomicAdd(&stats[0], (unsigned long long)st.evals);
      atomicAdd(&stats[1], (unsigned long long)st.steps);
      atomicAdd(&stats[2], (unsigned long long)st.forms);
      atomicAdd(&stats[3], (unsigned long long)st.screens);
      atomicAdd(&stats[4], (unsigned long long)n_blocks);
      atomicAdd(&stats[5], 1ull);
    }
  }
}


// Launch shape: a workgroup per 4 groups (x) and per rows_per_wg rows (y),
// rows per workgroup a multiple of 64 (one row per lane), about kSweepWgs
// workgroups (each builds its tables and factors its groups' H once).
inline dim3 sweep_grid(int64_t rows, int64_t k, int64_t* rows_per_wg) {
  const int64_t groups = k >> 4;
  const int64_t gx = (groups + kWaves - 1) / kWaves;
  int64_t rpw = (rows * gx + kSweepWgs - 1) / kSweepWgs;
  rpw = ((rpw + 63) / 64) * 64;
  if (rpw < kMinRowsPerWg) rpw = kMinRowsPerWg;
  if (rpw > kStageRows) rpw = kStageRows;                   // outputs staged in LDS (more workgroups instead)
  int64_t chunks = (rows + rpw - 1) / rpw;
  while (chunks > 65535) {
    rpw *= 2;
    chunks = (rows + rpw - 1) / rpw;
  }
  *rows_per_wg = rpw;
  return dim3((unsigned)gx, (unsigned)chunks, 1);
}

}  // namespace

}  // namespace nvfp4
