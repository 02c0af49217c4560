/*
 * nvfp4mi.h - C ABI of the MI355X (gfx950) NVFP4 post-training-quantization
 * hot path.
 *
 * NVFP4 stores a tensor as 4-bit E2M1 elements {0, +-0.5, +-1, +-1.5, +-2,
 * +-3, +-4, +-6}, one non-negative E4M3FN block scale per 16 consecutive
 * elements along the input-channel axis, and one FP32 tensor scale scale_2.
 * The value of element i of block b is e2m1(i) * RN_f32(e4m3(code_b) *
 * scale_2), cast to BF16 for use ("Coder390 NVFP4 校正（校准）方式" §2, format
 * paragraph; "NVFP4 量化流程说明" §2.2, §5.4).
 *
 * Common conventions
 * ------------------
 * - Every pointer argument is a DEVICE pointer (hipMalloc'ed or from a
 *   framework allocator) owned by the caller, unless stated otherwise.  The
 *   library keeps no pointer after a call returns and allocates no device
 *   memory of its own, except the hipBLASLt handle that
 *   nvfp4_quantlinear_forward creates on its first call on a device (kept
 *   until the process ends) and the static 16 MiB buffer of
 *   nvfp4_hessian_accum_noalloc (part of the library's device code, present
 *   on each device once the library runs there); scratch memory otherwise
 *   comes in as a caller-provided workspace.
 * - bf16 values are passed as uint16_t bit patterns.  Matrices are row-major;
 *   "ld" arguments are row strides in ELEMENTS.  Blocks of 16 run along the
 *   last (contiguous) axis.
 * - Packed E2M1 data: two codes per byte, element 2i in bits 0-3 and element
 *   2i+1 in bits 4-7; bit 3 of a code is the sign.  Block scales: one E4M3FN
 *   byte per block, row-major [rows][k/16].
 * - stream is a hipStream_t passed as void* (NULL = the default stream).  All
 *   work is enqueued on it asynchronously; outputs are valid once the stream
 *   has synchronised.  Kernel faults surface at that synchronisation.
 * - Arguments are validated on the host BEFORE any HIP call; on a validation
 *   error nothing is enqueued.  Functions return NVFP4_OK (0) or one of the
 *   NVFP4_ERR_* codes below; nvfp4_status_string() describes a code (for
 *   NVFP4_ERR_HIP it includes the HIP error text of the failing call on the
 *   calling thread).
 * - Buffers must not overlap unless stated (the cast rewrites its nibbles in
 *   place by design).  Calls are reentrant; concurrent calls must not share
 *   outputs or workspaces.
 * - Inputs are expected to be finite.  NaN/Inf inputs give unspecified codes.
 * - Test hook: the environment variable NVFP4MI_FORCE_EXACT, read at every
 *   launch of the quantizers, the sweep, the W4A4 Hessian and the fake QDQ,
 *   selects which of the certified E2M1 decision paths may be used (unset or
 *   0: all; 1: exact thresholds only; 2: not the one-float reciprocal; 3:
 *   neither of the uncorrected reciprocals).  Every path gives the same
 *   bits, so it changes speed, not results; the tests use it to run every
 *   case on each path.
 *
 * Rounding (readings of the pages, which name no rounding mode): every
 * encode rounds the exact real quotient once to nearest, ties to even, and
 * saturates at the format's largest finite value (6 for E2M1, 448 for E4M3);
 * a negative element that rounds to zero keeps its sign bit.
 */
#ifndef NVFP4MI_H
#define NVFP4MI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum nvfp4_status {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL_ARG = 1,     /* a required pointer is NULL                         */
  NVFP4_ERR_BAD_SHAPE = 2,    /* a size is negative, k % 16 != 0 (k % 32 for the
                                 cast), ld < k, or a product overflows int64       */
  NVFP4_ERR_MISALIGNED = 3,   /* a buffer or matrix row is not aligned as the
                                 function requires (16 bytes for bf16 rows)       */
  NVFP4_ERR_WORKSPACE = 4,    /* workspace smaller than the matching *_bytes() query */
  NVFP4_ERR_BAD_INPUT = 5,    /* an argument value is out of range (e.g. mats <= 0)  */
  NVFP4_ERR_HIP = 6,          /* a HIP launch or API call failed                     */
  NVFP4_ERR_SCRATCH_LIMIT = 7 /* the input needs more scratch than the static buffer
                                 of nvfp4_hessian_accum_noalloc holds               */
};

/* Text for a status code (static storage; for NVFP4_ERR_HIP the text of the
 * last HIP error seen on the calling thread). */
const char* nvfp4_status_string(int status);

/*
 * Step 1 of the per-Linear calibration, max calibration ("Coder390 NVFP4
 * 校正（校准）方式" §2 step 1), with the tensor-scale formula of "NVFP4
 * 量化流程说明" §3.4: amax = max |x| over n bf16 values and
 * scale_2 = RN_f32(amax / (6 * 448)).
 *
 * x          [n] bf16, contiguous, 16-byte aligned (n may be 0: amax = 0).
 * scale2_out device float[1]: receives scale_2.  Also used as the running
 *            accumulator, so it must not alias x.
 * amax_out   device float[1] or NULL: receives amax.
 * Errors: NULL_ARG (x with n > 0, scale2_out), BAD_SHAPE (n < 0),
 *         MISALIGNED (x; scale2_out or amax_out not 4-byte aligned), HIP.
 */
int nvfp4_compute_scale2(const uint16_t* x, int64_t n, float* scale2_out,
                         float* amax_out, void* stream);

/*
 * Step 1 for several tensors at once (a Linear's weight and its calibration
 * activations, the weights of one MLP, ...): for t < count, exactly what
 * nvfp4_compute_scale2(xs[t], ns[t], scale2_out + t, amax_out + t) gives,
 * in three kernel launches in all instead of three per tensor (the reduce
 * walks the tensors in turn, one atomic max per workgroup and tensor).
 *
 * xs, ns     HOST arrays of count entries: device pointers to bf16 tensors
 *            (contiguous, 16-byte aligned; NULL allowed where ns[t] == 0) and
 *            their element counts.  Read during the call only.
 * count      1 .. 16.
 * scale2_out device float[count]: receives the scale_2 values; also the
 *            running accumulators when amax_out is NULL, so it must not
 *            alias any input.
 * amax_out   device float[count] or NULL: receives the amax values (and is
 *            then the accumulator).
 * Errors: BAD_SHAPE (count out of range, ns[t] < 0), NULL_ARG (xs, ns,
 *         scale2_out, or xs[t] with ns[t] > 0), MISALIGNED (xs[t]; the
 *         output arrays not 4-byte aligned), HIP.
 */
int nvfp4_compute_scale2_batch(const uint16_t* const* xs, const int64_t* ns, int count,
                               float* scale2_out, float* amax_out, void* stream);

/*
 * Bytes of workspace nvfp4_hessian_accum and nvfp4_hessian_accum_fq need for
 * (tokens, k) (one size serves both); 0 when tokens == 0.  Returns 0 for
 * invalid sizes too (the accumulate call then reports the shape error).
 */
size_t nvfp4_hessian_workspace_bytes(int64_t tokens, int64_t k);

/*
 * Step 2, the local block-diagonal Hessian ("Coder390 NVFP4 校正（校准）方式"
 * §2 step 2): for every group g of 16 input channels,
 *   H[g] += sum_t x[t, 16g:16g+16]^T x[t, 16g:16g+16]
 * over the `tokens` rows of x, accumulated into H IN PLACE so a calibration
 * stream can be fed chunk by chunk.  Products of bf16 values are exact in
 * fp32; partial sums run in fp32 on MFMA over at most a few thousand tokens
 * and are then reduced in fp64 in a fixed order (bitwise reproducible).
 *
 * x          [tokens][ldx] bf16; columns 0..k-1 are used.
 * H          [k/16][16][16] float, in/out, 16-byte aligned.
 * amax_inout device float[1] or NULL: if given, it is raised to
 *            max(*amax_inout, max |x|) (step 1 fused into the same read of x).
 * workspace  16-byte aligned device buffer of at least
 *            nvfp4_hessian_workspace_bytes(tokens, k) bytes; contents are
 *            scratch.
 * Errors: NULL_ARG, BAD_SHAPE (tokens < 0, k <= 0, k % 16, ldx < k),
 *         MISALIGNED (x or ldx not 16-byte aligned rows; H or workspace not
 *         16-byte aligned; amax_inout not 4-byte aligned), WORKSPACE, HIP.
 */
int nvfp4_hessian_accum(const uint16_t* x, int64_t tokens, int64_t k, int64_t ldx,
                        float* H, float* amax_inout, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Step 2 ("Coder390 NVFP4 校正（校准）方式" §2 step 2) over several resident
 * chunks of one calibration stream in one call (for callers that keep a
 * stream's activations in device memory): for every group g,
 *   H[g] += sum over chunks c of X_c[:, 16g:16g+16]^T X_c[:, 16g:16g+16].
 * One accumulate launch per chunk, each into its own partial slots, then one
 * reduce over all of them, instead of a reduce per chunk.  The chunks are read
 * on `stream` after the call returns: keep them alive until that work is
 * done.  The fp32 partial sums are exactly those of one
 * nvfp4_hessian_accum call per chunk; they are then added in fp64 (chunk by
 * chunk, each in workgroup order) and H is rounded once, so the result may
 * differ from nvfp4_hessian_accum chunk by chunk in the last bits of H (it
 * rounds H once instead of once per chunk) and is bitwise reproducible.
 *
 * xs         HOST array of nchunks device pointers, each [tokens][ldx] bf16
 *            (columns 0..k-1 used; 16-byte aligned rows).  Read during the call.
 * nchunks    1 .. 64.
 * tokens, k, ldx, H, amax_inout, stream: as for nvfp4_hessian_accum (every
 *            chunk has the same shape; amax_inout is raised to the max |x|
 *            over all chunks).
 * workspace  16-byte aligned device buffer of at least
 *            nvfp4_hessian_chunks_workspace_bytes(tokens, k, nchunks) bytes
 *            (one chunk's partial slots per chunk, sized for either
 *            chunk-list call); scratch.
 * Errors: as for nvfp4_hessian_accum, plus BAD_SHAPE for nchunks out of range
 *         and NULL_ARG for xs or a NULL chunk.
 */
size_t nvfp4_hessian_chunks_workspace_bytes(int64_t tokens, int64_t k, int nchunks);
int nvfp4_hessian_accum_chunks(const uint16_t* const* xs, int nchunks, int64_t tokens,
                               int64_t k, int64_t ldx, float* H, float* amax_inout,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * nvfp4_hessian_accum without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same operation, kernels and results (bit for bit)
 * as nvfp4_hessian_accum; the fp32 partial slots live in a static device
 * buffer of 16 MiB inside the library instead (each GPU the library runs on
 * holds its own copy until the process ends), which fits every shape with
 * k <= 131072 and any token count.  The call allocates nothing; its first
 * call on a device looks up that device's buffer address
 * (hipGetSymbolAddress) with the device current.  All calls on one GPU share
 * the buffer: calls that overlap in time on one GPU (two host threads, or
 * two streams whose work may run concurrently) race and give wrong H; order
 * them on one stream or with events.  Nothing in the buffer needs clearing
 * between calls.
 * x, tokens, k, ldx, H, amax_inout, stream: as for nvfp4_hessian_accum.
 * Errors: as for nvfp4_hessian_accum without WORKSPACE, plus SCRATCH_LIMIT
 *         when nvfp4_hessian_workspace_bytes' plain-kernel share exceeds the
 *         16 MiB buffer (k > 131072), and HIP (also a failed address lookup).
 */
int nvfp4_hessian_accum_noalloc(const uint16_t* x, int64_t tokens, int64_t k, int64_t ldx,
                                float* H, float* amax_inout, void* stream);

/*
 * Step 2 for a W4A4 calibration, where the Linear's input passes through its
 * dynamic NVFP4 quantizer ("Coder390 NVFP4 校正（校准）方式" §3, the W4A4
 * tier; quantizer and two-level dequantization of "NVFP4 量化流程说明"
 * §3.4-§3.5): for every group g of 16 input channels,
 *   H[g] += sum_t xh[t, 16g:16g+16]^T xh[t, 16g:16g+16],
 *   xh = bf16 output of nvfp4_dequant(nvfp4_quantize_dynamic(x, scale2))
 * element for element, without writing the quantized activations to memory
 * (each 16-element block is quantized and dequantized in registers between
 * the load of x and the contraction).  Accumulation and reduction order are
 * those of nvfp4_hessian_accum, which it shares the workspace query with.
 *
 * x, tokens, k, ldx, H, workspace, workspace_bytes, stream: as for
 *            nvfp4_hessian_accum.
 * scale2     device float[1]: the activations' tensor scale (step 1 run
 *            beforehand, e.g. nvfp4_compute_scale2 over calibration inputs).
 * amax_inout device float[1] or NULL: raised to max(*amax_inout, max |x|)
 *            over the RAW (unquantized) input, for the next scale_2.
 * Errors: as for nvfp4_hessian_accum, plus NULL_ARG for scale2.
 */
int nvfp4_hessian_accum_fq(const uint16_t* x, int64_t tokens, int64_t k, int64_t ldx,
                           const float* scale2, float* H, float* amax_inout,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * nvfp4_hessian_accum_fq over several resident chunks in one call (the W4A4
 * tier of "Coder390 NVFP4 校正（校准）方式" §3; the W4A4 form of
 * nvfp4_hessian_accum_chunks): one accumulate launch per chunk
 * into its own partial slots, one fp64 reduce over all of them.
 * xs, nchunks, workspace (nvfp4_hessian_chunks_workspace_bytes serves both
 * chunk-list calls), chunk lifetime: as for nvfp4_hessian_accum_chunks;
 * scale2, H, amax_inout: as for nvfp4_hessian_accum_fq.
 * Errors: as for nvfp4_hessian_accum_chunks, plus NULL_ARG for scale2.
 */
int nvfp4_hessian_accum_fq_chunks(const uint16_t* const* xs, int nchunks, int64_t tokens,
                                  int64_t k, int64_t ldx, const float* scale2, float* H,
                                  float* amax_inout, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * Step 3, the Hessian-weighted block-scale sweep (fp8_scale_sweep,
 * "Coder390 NVFP4 校正（校准）方式" §2 step 3).  For every block b = (row r,
 * group g) of 16 weights w and every finite E4M3 code c in 0x00..0x7E:
 *   d_c  = RN_f32(e4m3(c) * scale_2)
 *   q    = E2M1 quantization of w / d_c (exact quotient, RNE, saturating;
 *          d_c = 0 quantizes to zero)
 *   cost = (w - q*d_c)^T H[g] (w - q*d_c)
 * and the code of least cost is kept (lowest code on ties).  Costs are
 * evaluated in fp32; the quantization itself is exact.  Codes whose cost is
 * provably larger than the best one found (Schur-complement lower bounds of
 * H[g], with a rounding margin) are skipped, which leaves the answer
 * unchanged.
 *
 * w       [rows][ldw] bf16, columns 0..k-1 (W of an nn.Linear: [out][in]).
 * H       [k/16][16][16] float, symmetric positive semidefinite (from
 *         nvfp4_hessian_accum); its upper triangle is read.
 * scale2  device float[1]: scale_2 of w (from nvfp4_compute_scale2).
 * packed  [rows][k/2] uint8 out: nibbles at the chosen codes.
 * codes   [rows][k/16] uint8 out: chosen E4M3 codes.
 * cost    [rows][k/16] float out or NULL: the fp32 cost of the chosen code.
 * Errors: NULL_ARG, BAD_SHAPE (rows < 0, k <= 0, k % 16, ldw < k),
 *         MISALIGNED (w rows), HIP.
 */
int nvfp4_scale_sweep(const uint16_t* w, int64_t rows, int64_t k, int64_t ldw,
                      const float* H, const float* scale2, uint8_t* packed,
                      uint8_t* codes, float* cost, void* stream);

/*
 * nvfp4_scale_sweep with an occupancy cap, for running the sweep beside an
 * HBM-bound kernel on another stream (e.g. nvfp4_hessian_accum of the next
 * calibration stream).  wgs_per_cu = 0: as nvfp4_scale_sweep (as many
 * workgroups per CU as fit); 1: at most one sweep workgroup per CU, by
 * reserving just over half of the CU's LDS per workgroup, which leaves the
 * rest of the LDS and about 260 VGPRs per SIMD to the other kernel.  Results
 * are identical to nvfp4_scale_sweep's.  The reservation is sized, and the
 * kernel's dynamic-LDS limit raised, once per device at its first capped call
 * (thread-safe).
 * Errors: as nvfp4_scale_sweep, plus BAD_INPUT (wgs_per_cu not 0 or 1, or a
 *         device index of 64 or more when capped).
 */
int nvfp4_scale_sweep_ex(const uint16_t* w, int64_t rows, int64_t k, int64_t ldw,
                         const float* H, const float* scale2, uint8_t* packed,
                         uint8_t* codes, float* cost, int wgs_per_cu, void* stream);

/*
 * Dynamic per-16 NVFP4 activation quantizer ("NVFP4 量化流程说明" §3.4-§3.5):
 * per block, amax_b = max |x| over the 16 elements, code =
 * RNE_sat(amax_b / (6 * scale_2)) on the E4M3 grid (raised to 0x01 if the
 * block is nonzero and that gives 0x00), then E2M1 quantization of every
 * element at d = RN_f32(e4m3(code) * scale_2).  One pass over x.
 *
 * x       [rows][ldx] bf16, columns 0..k-1.
 * scale2  device float[1]: the per-tensor scale (calibrated or from
 *         nvfp4_compute_scale2); 0 quantizes everything to zero.
 * packed  [rows][k/2] uint8 out;  codes [rows][k/16] uint8 out.
 * Errors: NULL_ARG, BAD_SHAPE, MISALIGNED, HIP.
 */
int nvfp4_quantize_dynamic(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx,
                           const float* scale2, uint8_t* packed, uint8_t* codes,
                           void* stream);

/*
 * Two-DequantizeLinear chain ("NVFP4 量化流程说明" §5.4): DQ1 d =
 * RN_f32(e4m3(code) * scale_2), DQ2 y = RN_f32(e2m1 * d), then a cast to
 * BF16 (nearest even).  Code 0x7F (NaN) gives NaN outputs.
 *
 * packed [rows][k/2] uint8, contiguous; codes [rows][k/16] uint8, contiguous;
 * scale2 device float[1];  out [rows][k] bf16, contiguous.
 * Errors: NULL_ARG, BAD_SHAPE (rows < 0, k <= 0, k % 16), MISALIGNED, HIP.
 */
int nvfp4_dequant(const uint8_t* packed, const uint8_t* codes, const float* scale2,
                  int64_t rows, int64_t k, uint16_t* out, void* stream);

/*
 * Closed-form MXFP4 -> NVFP4 cast ("从MXFP4到NVFP4：Model Optimizer混合精度格式
 * 转换完全攻略" §2-§3; "从校准到导出：DeepSeek-V4-Pro-0813-nvfp4-DSpark
 * 三阶段 NVFP4 量化流程实战", export stage).  The input holds `groups` groups of
 * `mats_per_group` MXFP4 matrices (e.g. an expert's w1 and w3) that share one
 * NVFP4 scale_2.  Per group, with k_j = e8m0_j - 127 and k_max its maximum:
 *   scale_2 = 2^(k_max - 8)             (global_amax = 6 * 448 * 2^(k_max - 8))
 *   MX block j with k_max - k_j <= 17:  both NVFP4 blocks get the E4M3 code of
 *                                       2^(k_j - k_max + 8); nibbles untouched
 *   otherwise (fallback):               each 16-element half is requantized from
 *                                       its data with the dynamic quantizer's
 *                                       rule (block amax, code raised to 0x01)
 * E8M0 code 255 (NaN) is left out of k_max; its blocks get code 0x7F (NaN)
 * and keep their nibbles.
 *
 * packed   [groups][mats][rows][k/2] uint8, IN/OUT: only fallback blocks are
 *          rewritten.
 * e8m0     [groups][mats][rows][k/32] uint8.
 * codes_out  [groups][mats][rows][k/16] uint8 out.
 * scale2_out [groups] float out (also used as scratch during the call).
 * fallback_blocks_out [groups] int64 out or NULL: number of 32-element MX
 *          blocks per group that took the fallback (0 = lossless group).
 * Errors: NULL_ARG, BAD_SHAPE (sizes <= 0, k % 32), BAD_INPUT, MISALIGNED
 *         (packed/e8m0/codes_out not 16-byte aligned, scale2_out not 4-byte
 *         or fallback_blocks_out not 8-byte aligned), HIP.
 */
int mxfp4_to_nvfp4_cast(uint8_t* packed, const uint8_t* e8m0, int64_t groups,
                        int64_t mats_per_group, int64_t rows, int64_t k,
                        uint8_t* codes_out, float* scale2_out,
                        int64_t* fallback_blocks_out, void* stream);

/*
 * FP8 E4M3 tier with per-tensor static scales: the W8A8 layers of the mixed
 * W4A4+W8A8 tier ("Coder390 NVFP4 校正（校准）方式" §3, layer table: attention
 * projections in FP8 E4M3, activations with static scales from calibration).
 * The page gives no formula; the scale is max calibration over the E4M3 range
 * (the NVFP4 tensor scale of "NVFP4 量化流程说明" §3.4 without the E2M1
 * factor 6) and the encode rounds the exact quotient like every encode here.
 */

/*
 * s = RN_f32(amax / 448), amax = max |x| over n bf16 values.
 * x [n] bf16, contiguous, 16-byte aligned (n may be 0: s = 0).
 * scale_out device float[1] (also the running accumulator: must not alias x);
 * amax_out device float[1] or NULL.
 * Errors: NULL_ARG (x with n > 0, scale_out), BAD_SHAPE (n < 0), MISALIGNED
 *         (x; scale_out or amax_out not 4-byte aligned), HIP.
 */
int fp8e4m3_compute_scale(const uint16_t* x, int64_t n, float* scale_out,
                          float* amax_out, void* stream);

/*
 * q[r][c] = E4M3FN code of x[r][c] / s: the exact quotient rounded to nearest
 * with ties to even, saturated at 448, sign in bit 7 (a negative value that
 * rounds to zero gives 0x80).  s = 0 maps 0 to 0 and any other value to
 * +-448.  Inputs are taken as finite.
 * x     [rows][ldx] bf16, columns 0..k-1; rows 16-byte aligned (ldx % 8 == 0).
 * scale device float[1], s >= 0 (e.g. from fp8e4m3_compute_scale).
 * q     [rows][k] uint8, contiguous, 8-byte aligned.
 * Errors: NULL_ARG, BAD_SHAPE (rows < 0, k <= 0, k % 8, ldx < k, overflow),
 *         MISALIGNED, HIP.
 */
int fp8e4m3_quantize(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx,
                     const float* scale, uint8_t* q, void* stream);

/*
 * out[r][c] = RN_bf16(RN_f32(e4m3(q[r][c]) * s)); codes 0x7F/0xFF give NaN.
 * q [rows][k] uint8, contiguous, 8-byte aligned; out [rows][k] bf16,
 * contiguous, 16-byte aligned.
 * Errors: NULL_ARG, BAD_SHAPE (k % 8 and as above), MISALIGNED, HIP.
 */
int fp8e4m3_dequant(const uint8_t* q, const float* scale, int64_t rows, int64_t k,
                    uint16_t* out, void* stream);

/*
 * Block-Hadamard rotation of the input channels under the local-Hessian sweep
 * ("FP4量化技术概述：从理论到硬件实现" §3.1, MR-GPTQ: the block Hadamard
 * transform fused into the weights, W' = W H, activations rotated online).
 * Per NVFP4 group of 16 input channels R_g = H16 / 4 (Sylvester order), so
 * X W^T = (X R)(W R)^T; the rotated input's local Hessian is R_g^T H_g R_g,
 * and the sweep of (W R, R^T H R) has the cost of the un-rotated error, so
 * its costs compare directly with the plain sweep's.
 */

/*
 * out[r][16g + i] = RN_bf16(((x[r][16g:16g+16] H16) / 4)_i): the Sylvester
 * butterfly in fp64 (exact unless a block spans more than 2^41), rounded once
 * to bf16 (nearest even).  Rotates weights (W R) and activations (X R) alike.
 * x   [rows][ldx] bf16, columns 0..k-1; out [rows][ldo] bf16.  Rows 16-byte
 *     aligned (ldx, ldo multiples of 8).  out may be x itself with ldo == ldx
 *     (in place); otherwise the two must not overlap.
 * Errors: NULL_ARG, BAD_SHAPE (k % 16, ld < k, sizes), MISALIGNED, HIP.
 */
int nvfp4_block_hadamard(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx,
                         uint16_t* out, int64_t ldo, void* stream);

/*
 * H_out[g] = RN_f32(R_g^T H[g] R_g) for g < groups, in fp64.  H and H_out are
 * [groups][16][16] float; H_out may be H (in place), otherwise no overlap.
 * Errors: NULL_ARG, BAD_SHAPE (groups < 0), MISALIGNED (H or H_out not
 *         4-byte aligned), HIP.
 */
int nvfp4_hessian_hadamard(const float* H, int64_t groups, float* H_out, void* stream);

/*
 * NVFP4 block fake QDQ of an activation tensor, the QuantLinear input
 * quantizer of "NVFP4 量化流程说明" §2.2: out = the bf16 result of
 * nvfp4_dequant(nvfp4_quantize_dynamic(x, scale2)) element for element, in one
 * pass without the packed intermediate.
 * x [rows][ldx] bf16 and out [rows][ldo] bf16, columns 0..k-1, rows 16-byte
 * aligned; scale2 device float[1].
 * Errors: NULL_ARG, BAD_SHAPE (k % 16, ld < k, sizes), MISALIGNED, HIP.
 */
int nvfp4_fakequant(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx,
                    const float* scale2, uint16_t* out, int64_t ldo, void* stream);

/*
 * Bytes of workspace nvfp4_quantlinear_forward needs (0 for invalid sizes).
 */
size_t nvfp4_quantlinear_workspace_bytes(int64_t tokens, int64_t k);

/*
 * Fake-quant QuantLinear forward of the calibration pass ("NVFP4 量化流程说明"
 * §2.2, §2.4: x -> input quantizer (block fake QDQ) -> matmul with the
 * fake-quantized weight, still a bf16 GEMM):
 *   y[t][o] = RN_bf16( sum_k xh[t][k] w[o][k] ), fp32 accumulation,
 * xh = nvfp4_fakequant(x, x_scale2).  w is the fake-quantized weight in bf16
 * (nvfp4_dequant of the swept NVFP4 weight, computed once per layer).  The
 * fake QDQ is one kernel of this library into the workspace; the product is
 * a plain bf16 GEMM through hipBLASLt (fp32 compute; its summation order is
 * hipBLASLt's).  The first call on a device creates a hipBLASLt handle (kept
 * until the process ends).  The first call for each new shape times up to 16
 * of hipBLASLt's candidate algorithms on `stream` and keeps the fastest, so
 * that call synchronises the stream; under graph capture it takes the first
 * candidate untimed.
 * x [tokens][ldx] bf16; w [out_features][ldw] bf16; y [tokens][ldy] bf16;
 * rows 16-byte aligned.  workspace: 256-byte aligned device buffer of at
 * least nvfp4_quantlinear_workspace_bytes(tokens, k) bytes (scratch).
 * Errors: NULL_ARG, BAD_SHAPE (k % 16, ld < k, out_features <= 0, sizes),
 *         MISALIGNED, WORKSPACE, HIP (also hipBLASLt failures).
 */
int nvfp4_quantlinear_forward(const uint16_t* x, int64_t tokens, int64_t k, int64_t ldx,
                              const float* x_scale2, const uint16_t* w, int64_t out_features,
                              int64_t ldw, uint16_t* y, int64_t ldy, void* workspace,
                              size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4MI_H */
