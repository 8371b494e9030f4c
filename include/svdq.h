/*
 * svdq.h -- C ABI of the SVDQuant linear layer for AMD Instinct MI355X (gfx950).
 *
 * The layer computes, for X (b x m) and a prepared weight W (m x n),
 *
 *     Y = Q(X diag(lambda)^-1) Q(R) + (X diag(lambda)^-1 L1) L2  (+ bias)
 *
 * Sources (cited by section / equation / algorithm; no text is quoted):
 *   [Review]   "SVDQuant: How a Small High-Precision Branch Makes 4-Bit
 *              Diffusion Practical" -- technical review of arXiv:2411.05007v4.
 *   [Nunchaku] "SVDQuant: 4-bit Quantization Enables Efficient Diffusion Model
 *              Inference on Consumer GPUs", section "Nunchaku".
 *
 * Conventions shared by every entry point
 *   - All matrices are row-major; dimensions are int32; 0 <= b <= SVDQ_MAX_DIM,
 *     1 <= m, n <= SVDQ_MAX_DIM.
 *   - The quantization group is 64 input channels (argument `group` must be
 *     SVDQ_GROUP) and m must be a multiple of 64 ([Review] sec. 8: INT4 uses
 *     group 64 on both operands with 16-bit scales).
 *   - INT4 codes are symmetric in [-7, 7] ([Review] sec. 2.2, Eq.(1)); two codes
 *     per byte, even channel in the low nibble ([Nunchaku]).
 *   - Packed code tensors are GROUP-MAJOR: for group g (channels 64g..64g+63)
 *     and row (or column) r, one 32-byte record holds the 64 codes; byte t of
 *     the record = code[64g+2t] | code[64g+2t+1] << 4.  A tensor of R rows is
 *     laid out [m/64][R][32].
 *   - Scales are IEEE fp16 bit patterns, bf16 tensors are bf16 bit patterns
 *     (uint16_t); fp32 is IEEE float.
 *   - "HOST" entry points take host pointers and run synchronously on the CPU
 *     (offline preparation, [Review] sec. 5 Algorithm 1).  "DEVICE" entry points
 *     take device pointers, validate on the host, then enqueue HIP kernels on
 *     `stream` (a hipStream_t; NULL = default stream) and return without
 *     synchronising ([Review] sec. 6.1 Algorithm 2).
 *   - Ownership: the caller allocates and frees every buffer.  The library
 *     never allocates device memory and keeps no pointer after a call returns.
 *   - Errors: every argument is checked BEFORE any HIP call or any write; on an
 *     error nothing is launched, no output is touched, and a nonzero
 *     svdq_status is returned.  svdq_last_error() gives a message (per
 *     thread).  Faults inside a kernel surface at the caller's next
 *     synchronisation, as usual for HIP.
 *   - Device pointers must be 16-byte aligned unless stated otherwise.
 *   - Every entry point is reentrant; the only library state is the per-thread
 *     error message.
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum svdq_status {
  SVDQ_OK = 0,
  SVDQ_ERR_INVALID_ARG = 1,    /* null pointer, bad dimension, alpha outside [0, 1] */
  SVDQ_ERR_UNSUPPORTED = 2,    /* group != 64, m % 64 != 0, rank above the limit */
  SVDQ_ERR_ALIGNMENT = 3,      /* device pointer not 16-byte aligned */
  SVDQ_ERR_NONFINITE = 4,      /* NaN / Inf in a preparation input */
  SVDQ_ERR_NO_CONVERGENCE = 5, /* truncated SVD did not converge */
  SVDQ_ERR_WORKSPACE = 6,      /* workspace missing or too small */
  SVDQ_ERR_HIP = 7,            /* a HIP launch or runtime call failed */
  SVDQ_ERR_IO = 8              /* a layer file could not be written or read, or is not valid */
} svdq_status;

enum { SVDQ_OUT_BF16 = 0, SVDQ_OUT_F32 = 1 };

#define SVDQ_GROUP 64
#define SVDQ_MAX_RANK 256
/* Largest b, m and n accepted (device kernels address a group's records and a
 * rank block of L1 with 32-bit buffer offsets). */
#define SVDQ_MAX_DIM (1 << 22)

/*
 * A prepared layer on the device ([Review] sec. 5 Algorithm 1, step 9: the
 * stored factors, quantized residual, scales and transform).  Every pointer is
 * DEVICE memory owned by the caller.
 *   m, n        input / output features; m % 64 == 0.
 *   rank        width r of the protected branch, 0 <= r <= SVDQ_MAX_RANK.
 *   group       must be 64.
 *   smooth_inv  fp32 [m]: 1/lambda (the runtime half of Eq.(3), X~ = X D^-1),
 *               or NULL for no smoothing.
 *   qw          INT4 codes of the residual R, group-major [m/64][n][32].
 *   wscale      fp16 [m/64][n]: one scale per (group, output column).
 *   l1          bf16 [rank][m]: L1 TRANSPOSED (each of the r columns of L1 is
 *               contiguous).  NULL iff rank == 0.
 *   l2          bf16 [n][rank]: L2 TRANSPOSED (the r coefficients of each output
 *               column are contiguous; any alignment).  NULL iff rank == 0.
 *   bias        bf16 [n] added before the store ([Review] Algorithm 2 step 8),
 *               or NULL (any alignment).
 */
typedef struct svdq_layer {
  int32_t m, n, rank, group;
  const float* smooth_inv;
  const uint8_t* qw;
  const uint16_t* wscale;
  const uint16_t* l1;
  const uint16_t* l2;
  const uint16_t* bias;
} svdq_layer;

/* ---------------------------------------------------------------------------
 * HOST: offline preparation of one layer  ([Review] sec. 3.1 Eq.(3)-(4),
 * sec. 5 Eq.(10) and Algorithm 1 steps 2-5).
 *
 *   W         fp32 [m][n], the original weight (finite).
 *   act_amax  fp32 [m] calibration maxima max_i |X_ik| (finite, >= 0), or NULL
 *             for no smoothing (lambda = 1).
 *   alpha     migration strength in [0, 1] (0.5 in the configurations here).
 *   Computes lambda_k = a_k^alpha / w_k^(1-alpha) with w_k = max_j |W_kj| in
 *   fp64 (lambda_k = 1 where a_k or w_k is 0), W~ = diag(lambda) W, a rank-r
 *   truncated SVD W~ ~ L1 L2 with Sigma folded into L1, bf16 factors, the
 *   residual R = W~ - L1 L2 in fp64 using the bf16 factors, and its INT4 group
 *   quantization with fp16 scales s = fp16(fl32(amax / 7)).
 *   Outputs (HOST buffers, caller-allocated, sizes as in svdq_layer):
 *     qw [m/64][n][32], wscale [m/64][n], l1 [rank][m], l2 [n][rank],
 *     lambda fp32 [m], smooth_inv fp32 [m] (= fl32(1 / lambda)),
 *     residual fp32 [m][n] (nullable: the fp32 R that was quantized).
 *   l1 / l2 may be NULL iff rank == 0.  1 <= rank <= min(m, n, SVDQ_MAX_RANK)
 *   or rank == 0.  Uses fp64 and all host cores; returns
 *   SVDQ_ERR_NO_CONVERGENCE if the SVD iteration fails.
 * ------------------------------------------------------------------------- */
int svdq_prepare_weights(const float* W, const float* act_amax, int m, int n, int rank,
                         int group, float alpha, uint8_t* qw, uint16_t* wscale, uint16_t* l1,
                         uint16_t* l2, float* lambda, float* smooth_inv, float* residual);

/* HOST: offline preparation with candidate search and refinement ([Review]
 * sec. 5 Algorithm 1 steps 2-8).  For each migration strength alphas[a] the
 * layer is built as in svdq_prepare_weights (steps 2-5); then `iters` times
 * the factors are re-fitted to the part of W~ the quantized residual leaves
 * out, L1 L2 <- rank-r SVD of (W~ - Q(R)), and R and Q(R) are formed again
 * (steps 6-7).  Every candidate (alpha, refinement step) is scored by its
 * layer-output error on calibration activations, ||Y(X_cal) - X_cal W||_F /
 * ||X_cal W||_F with Y the quantized layer exactly as the device computes it
 * (in fp64 on the host), and the first candidate with the lowest error is
 * returned (step 8).
 *   x_cal     bf16 [b_cal][m] calibration rows (host), b_cal >= 1.
 *   alphas    n_alpha (1..64) values in [0, 1]; iters in [0, 16].
 *   Outputs as svdq_prepare_weights, plus (each nullable) alpha_out: the
 *   chosen alpha; iter_out: its refinement step (0 = none); rel_err_out: its
 *   relative output error.  With alphas = {alpha}, iters = 0 the layer is
 *   identical to svdq_prepare_weights(..., alpha, ...). */
int svdq_prepare_weights_refined(const float* W, const float* act_amax, const uint16_t* x_cal, int b_cal,
                                 int m, int n, int rank, int group, const float* alphas, int n_alpha,
                                 int iters, uint8_t* qw, uint16_t* wscale, uint16_t* l1, uint16_t* l2,
                                 float* lambda, float* smooth_inv, float* residual, float* alpha_out,
                                 int* iter_out, double* rel_err_out);

/* ---------------------------------------------------------------------------
 * HOST: stored layers ([Review] sec. 5 Algorithm 1 step 9: keep the protected
 * factors, the quantized residual, its scales and the smoothing transform, so
 * a layer is prepared once and loaded afterwards).
 *
 * A prepared INT4 layer as HOST arrays in the layouts of svdq_layer
 * (caller-owned; what svdq_prepare_weights and svdq_append_lora produce):
 *   lambda, smooth_inv fp32 [m]; qw [m/64][n][32]; wscale fp16 [m/64][n];
 *   l1 bf16 [rank][m], l2 bf16 [n][rank] (NULL iff rank == 0); bias bf16 [n]
 *   or NULL; alpha: the migration strength it was prepared with (recorded).
 * ------------------------------------------------------------------------- */
typedef struct svdq_host_layer {
  int32_t m, n, rank, group;
  float alpha;
  const float* lambda;
  const float* smooth_inv;
  const uint8_t* qw;
  const uint16_t* wscale;
  const uint16_t* l1;
  const uint16_t* l2;
  const uint16_t* bias;
} svdq_host_layer;

/* Write `layer` to `path` (versioned binary file: a 64-byte header with the
 * dimensions, rank, group, alpha, a bias flag and an FNV-1a checksum of the
 * payload, then the arrays in the order above).  The file is written under a
 * temporary name and renamed, so readers never see a partial file.
 * SVDQ_ERR_INVALID_ARG / SVDQ_ERR_UNSUPPORTED for bad arguments (as
 * svdq_prepare_weights), SVDQ_ERR_IO if the file cannot be written. */
int svdq_save_layer(const char* path, const svdq_host_layer* layer);

/* Read the header of a layer file: m, n, rank, has_bias (0/1), alpha
 * (nullable).  SVDQ_ERR_IO if the file is missing, not a layer file, of
 * another version, or its payload size does not match its dimensions. */
int svdq_load_layer_info(const char* path, int32_t* m, int32_t* n, int32_t* rank, int32_t* has_bias,
                         float* alpha);

/* Read a layer file into caller HOST buffers sized from svdq_load_layer_info
 * (l1 / l2 may be NULL iff rank == 0, bias iff none is stored).  The buffers
 * are written only if the whole payload is present and its checksum matches;
 * otherwise SVDQ_ERR_IO and the buffers are untouched. */
int svdq_load_layer(const char* path, float* lambda, float* smooth_inv, uint8_t* qw, uint16_t* wscale,
                    uint16_t* l1, uint16_t* l2, uint16_t* bias);

/* HOST: the INT4 group quantization step alone ([Review] Algorithm 1 step 5 with
 * Eq.(1)): R fp32 [m][n] -> qw [m/64][n][32], wscale fp16 [m/64][n]. */
int svdq_quantize_residual(const float* R, int m, int n, int group, uint8_t* qw,
                           uint16_t* wscale);

/* HOST: attach an additive adapter W += scale * A B without re-quantizing
 * ([Review] sec. 7, Eq.(13)).  In smoothed coordinates the adapter is (D A) B,
 * so the branch widens to
 *     L1' = [L1 | bf16(diag(lambda) A)],   L2' = [L2 ; bf16(scale B)],
 * rank' = rank + k; qw and wscale are untouched.
 *   l1 bf16 [rank][m], l2 bf16 [n][rank] (may be NULL iff rank == 0),
 *   lambda fp32 [m] or NULL (= 1), A fp32 [m][k], B fp32 [k][n], k >= 1,
 *   rank + k <= SVDQ_MAX_RANK.
 *   Outputs: l1_out bf16 [rank+k][m], l2_out bf16 [n][rank+k]. */
int svdq_append_lora(const uint16_t* l1, const uint16_t* l2, int m, int n, int rank,
                     const float* lambda, const float* A, const float* B, int k, float scale,
                     uint16_t* l1_out, uint16_t* l2_out);

/* DEVICE: calibration statistic a_k = max_i |X_ik| over one batch of layer
 * inputs ([Review] sec. 3.1 Eq.(4) statistics; Algorithm 1 step 1).
 *   x bf16 [b][m]; amax fp32 [m].  accumulate != 0 folds the batch into the
 *   existing amax (max of both), otherwise amax is overwritten.  m % 8 == 0. */
int svdq_calibrate_act_amax(const uint16_t* x, int b, int m, float* amax, int accumulate,
                            void* stream);

/* Bytes of device workspace svdq_quantize_act_lowrank_down needs when it
 * splits the channel groups of a row block over several workgroups: the
 * partial sums of Z, added in split order by a second kernel (0 when no
 * split is needed).  The contents need no initialisation; calls that overlap
 * in time must not share it. */
size_t svdq_act_workspace_size(int b, int m, int rank);

/* DEVICE: fused activation quantization + low-rank down-projection
 * ([Review] sec. 6.1 Algorithm 2 steps 1-3; Fig. 4 first fused pair).
 * Each 64-channel group of every row is read once:
 *     x~ = bf16(fl32(x * smooth_inv))             (Eq.(3), X~ = X D^-1)
 *     ascale = fp16(fl32(max|x~| / 7)),  qx = clamp(round(x~ / ascale), -7, 7)  (Eq.(1))
 *     z = x~ L1 (fp32 accumulation)
 *   x bf16 [b][m]; smooth_inv fp32 [m] or NULL; l1 bf16 [rank][m] (NULL iff
 *   rank == 0).  Outputs: qx group-major [m/64][b][32], ascale fp16 [m/64][b]
 *   (any alignment), z fp32 [b][rank] (NULL iff rank == 0).
 *   workspace: device, >= svdq_act_workspace_size(b, m, rank) bytes (may be
 *   NULL when that is 0). */
int svdq_quantize_act_lowrank_down(const uint16_t* x, int b, int m, int rank, int group,
                                   const float* smooth_inv, const uint16_t* l1, uint8_t* qx,
                                   uint16_t* ascale, float* z, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Bytes of device workspace svdq_gemm_w4a4_lowrank_up may need for an output
 * of b x n with m input channels: the partial tiles of its split-K schedule
 * (an upper bound valid on every gfx950 device and GEMM setting; 0 when m has
 * too few channel groups to split). */
size_t svdq_gemm_workspace_size(int b, int n, int m);

/* Operand settings of the GEMM kernels, for svdq_gemm_schedule. */
enum { SVDQ_GEMM_INT4 = 0, SVDQ_GEMM_W8A8 = 1, SVDQ_GEMM_FP4 = 2 };

/* HOST (queries the current device's CU count; no launch): the schedule the
 * GEMM kernel of `setting` (SVDQ_GEMM_*) would use for an output of b x n with
 * m input channels ([Nunchaku]: one kernel per fused pair; the split of output
 * tiles over workgroups is this library's own).  Writes info[0] = output tiles
 * (128 x 128; 128 x 64 in the INT4 setting when the 128 x 128 tiles would not
 * fill one round of workgroups), info[1] = workgroups launched, info[2] = split workgroups
 * (each computes one piece of a tile's channel groups, and a reduction kernel
 * then adds the pieces; 0 when every workgroup computes one whole tile),
 * info[3] = tiles split (info[2] / info[3] pieces each), info[4] = resident
 * workgroups per CU of the kernel chosen.
 * info: host, 5 ints, owned by the caller.  On an error info is
 * untouched: SVDQ_ERR_INVALID_ARG for a null info, an unknown setting, b < 0
 * or n < 1; SVDQ_ERR_UNSUPPORTED for b, n or m above SVDQ_MAX_DIM, m not a
 * positive multiple of 64, or m > SVDQ_W8A8_MAX_M with SVDQ_GEMM_W8A8. */
int svdq_gemm_schedule(int b, int n, int m, int setting, int* info);

/* DEVICE: fused W4A4 GEMM + low-rank up-projection ([Review] sec. 6.1
 * Algorithm 2 steps 4-8; Eq.(7)):
 *     isum[i,j,g] = sum_{k in g} qx[i,k] qw[k,j]          (exact integer)
 *     Y[i,j] = sum_g ascale[g,i] wscale[g,j] isum[i,j,g] + (bf16(z) L2)[i,j] + bias[j]
 *   qx, ascale, z as produced by svdq_quantize_act_lowrank_down (z NULL iff
 *   layer->rank == 0; z any 4-byte alignment); y [b][n] in y_dtype
 *   (SVDQ_OUT_BF16, round-to-nearest-even, or SVDQ_OUT_F32); y needs only
 *   element alignment.  layer->smooth_inv and layer->l1 are not used.
 *   workspace: device, 16-byte aligned, >= svdq_gemm_workspace_size(b, n, m)
 *   bytes.  Its contents need no initialisation (every slot read is first
 *   written by the same call), and calls that overlap in time must not share
 *   it; a launch captured in a HIP graph may be replayed (stream-ordered) on
 *   the same workspace.  A split schedule launches two kernels on `stream`
 *   (the GEMM, then the reduction of the split tiles).  Per-group sums, and
 *   the pieces of a split tile, are added in a fixed order that depends only
 *   on the shape and the device's CU count, so results are deterministic. */
int svdq_gemm_w4a4_lowrank_up(const uint8_t* qx, const uint16_t* ascale, const float* z,
                              const svdq_layer* layer, int b, void* y, int y_dtype, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Bytes of device workspace svdq_linear needs (qx, ascale, Z and its split
 * partial sums, and the GEMM's workspace). */
size_t svdq_linear_workspace_size(int b, int m, int n, int rank, int group);

/* DEVICE: the whole layer = the two fused kernels back to back on `stream`
 * ([Review] sec. 6.1 Algorithm 2 steps 1-8).  x bf16 [b][m]; y [b][n] in
 * y_dtype; workspace >= svdq_linear_workspace_size(b, m, n, rank, group)
 * bytes, 256-byte aligned, not shared by calls that overlap in time.  Runs
 * exactly the kernels of the two entry points above, so its output is
 * bit-identical to theirs. */
int svdq_linear(const uint16_t* x, const svdq_layer* layer, int b, void* y, int y_dtype,
                void* workspace, size_t workspace_bytes, void* stream);

/* DEVICE: svdq_linear without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  It runs exactly svdq_linear's kernels
 * (bit-identical output) on a workspace taken from device scratch memory that
 * the library holds in a static device array of
 * svdq_linear_noalloc_max_workspace() bytes (128 MiB) on each GPU it runs
 * on, until the process ends.  It calls no allocator.
 *   Arguments as svdq_linear.  Returns SVDQ_ERR_WORKSPACE, before any launch,
 *   when svdq_linear_workspace_size(b, m, n, rank, 64) exceeds the scratch.
 *   Every call on one GPU shares that GPU's scratch: calls that overlap in
 *   time on one GPU (on different streams, or from several threads without
 *   ordering) race and give undefined results; stream-ordered calls are safe.
 *   The scratch keeps whatever the last call left; no part of it needs
 *   clearing (every byte a call reads it first writes). */
int svdq_linear_noalloc(const uint16_t* x, const svdq_layer* layer, int b, void* y, int y_dtype, void* stream);
size_t svdq_linear_noalloc_max_workspace(void);

/* Static description of a status code. */
const char* svdq_status_string(int status);

/* Message describing the last error raised on the calling thread ("" if none). */
const char* svdq_last_error(void);

/* ABI version of this header (major * 100 + minor). */
int svdq_abi_version(void);

/* TEST HOOK, not for production use: caps the iterations the preparation's
 * eigen-solver (the Rayleigh-Ritz step of the truncated SVD) may spend on one
 * eigenvalue; limit < 0 restores the default (60).  With a limit of 0 every
 * preparation of a layer with rank > 0 fails with SVDQ_ERR_NO_CONVERGENCE, so
 * tests can reach that error path.  Process-wide (not per thread); returns the
 * previous limit. */
int svdq_test_set_svd_iteration_limit(int limit);

/* DEVICE: the same layer WITHOUT the Nunchaku fusion, for measuring what the
 * fusion saves ([Review] sec. 6.1: a separate down-projection reads X again
 * and a separate up-projection writes a second b x n output that must be
 * added; [Nunchaku]: the two fused kernel pairs).  Five launches on `stream`:
 * activation quantization alone, the W4A4 product (+ bias) into y, the
 * down-projection alone (x read again), the up-projection alone into a b x n
 * tensor of y's type in the workspace, and y += that tensor.  The result is
 * the same layer as svdq_linear up to rounding: the two partial outputs are
 * each rounded to y_dtype before the addition.  Arguments as svdq_linear; y
 * must be 16-byte aligned; workspace >= svdq_linear_unfused_workspace_size(...)
 * bytes, 256-byte aligned, not shared by calls that overlap in time. */
size_t svdq_linear_unfused_workspace_size(int b, int m, int n, int rank, int group);
int svdq_linear_unfused(const uint16_t* x, const svdq_layer* layer, int b, void* y, int y_dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ===========================================================================
 * The 8-bit setting ([Review] sec. 8: W8A8 keeps the smoothing and the
 * low-rank branch, rank 16 there, with one scale per token of X~ and one per
 * output channel of R).
 *   - INT8 codes are symmetric in [-127, 127], one per byte (int8_t): for a
 *     row v of X~ (or a column of R), s = fp16(fl32(max|v| / 127)) saturated,
 *     code = clamp(round_half_even(fl32(v / s)), -127, 127), 0 where s = 0
 *     (the INT4 quantizer of [Review] sec. 2.2 Eq.(1) with 127 for 7).
 *   - Code tensors are GROUP-MAJOR in 64-byte records: for channels
 *     64g..64g+63 and row (or column) r, one record holds their 64 codes in
 *     channel order; a tensor of R rows is laid out [m/64][R][64].
 *   - m <= SVDQ_W8A8_MAX_M, so the exact integer products over all m channels
 *     (at most 127^2 m in magnitude) fit in int32.
 * Other conventions as above.
 * ========================================================================= */
#define SVDQ_W8A8_MAX_M 131072

/* A prepared 8-bit layer on the device (caller-owned DEVICE pointers).
 *   m, n, rank  as in svdq_layer (m % 64 == 0, m <= SVDQ_W8A8_MAX_M).
 *   smooth_inv  fp32 [m] or NULL; l1 bf16 [rank][m]; l2 bf16 [n][rank]
 *               (any alignment); bias bf16 [n] or NULL: as in svdq_layer.
 *   qw          INT8 codes of R, group-major [m/64][n][64].
 *   wscale      fp16 [n]: one scale per output column (any 2-byte alignment). */
typedef struct svdq_w8a8_layer {
  int32_t m, n, rank;
  const float* smooth_inv;
  const int8_t* qw;
  const uint16_t* wscale;
  const uint16_t* l1;
  const uint16_t* l2;
  const uint16_t* bias;
} svdq_w8a8_layer;

/* HOST: offline preparation of an 8-bit layer: steps 2-4 of [Review]
 * Algorithm 1 exactly as svdq_prepare_weights (lambda, W~, bf16 rank-r
 * factors, R = W~ - L1 L2), then R quantized per output column to INT8.
 * Outputs (HOST, caller-allocated): qw [m/64][n][64], wscale fp16 [n],
 * l1 [rank][m], l2 [n][rank], lambda, smooth_inv fp32 [m], residual fp32
 * [m][n] (nullable).  Errors as svdq_prepare_weights; m <= SVDQ_W8A8_MAX_M. */
int svdq_w8a8_prepare_weights(const float* W, const float* act_amax, int m, int n, int rank,
                              float alpha, int8_t* qw, uint16_t* wscale, uint16_t* l1,
                              uint16_t* l2, float* lambda, float* smooth_inv, float* residual);

/* Bytes of device workspace svdq_w8a8_quantize_act_lowrank_down needs (the
 * split partial sums of Z, as svdq_act_workspace_size; 0 when none). */
size_t svdq_w8a8_act_workspace_size(int b, int m, int rank);

/* DEVICE: per-token activation quantization + low-rank down-projection.
 *     x~ = bf16(fl32(x * smooth_inv))
 *     ascale[i] = fp16(fl32(max_k |x~[i,k]| / 127)),  qx = the INT8 codes of x~
 *     z = x~ L1 (fp32 accumulation; the same kernel and summation order as
 *       svdq_quantize_act_lowrank_down, so z is bit-identical to its z)
 * A row's scale needs the whole row, so the codes come from a kernel of their
 * own (one wave per row) and x is read a second time for z.
 *   x bf16 [b][m]; outputs qx [m/64][b][64], ascale fp16 [b] (any 2-byte
 *   alignment), z fp32 [b][rank] (NULL iff rank == 0).  Other arguments as
 *   svdq_quantize_act_lowrank_down. */
int svdq_w8a8_quantize_act_lowrank_down(const uint16_t* x, int b, int m, int rank,
                                        const float* smooth_inv, const uint16_t* l1, int8_t* qx,
                                        uint16_t* ascale, float* z, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* Bytes of device workspace svdq_w8a8_gemm_lowrank_up may need (int32 partial
 * tiles of its split-K schedule and one fp32 low-rank tile per split tile; the
 * bound of svdq_gemm_workspace_size). */
size_t svdq_w8a8_gemm_workspace_size(int b, int n, int m);

/* DEVICE: 8-bit GEMM + low-rank up-projection:
 *     isum[i,j] = sum_k qx[i,k] qw[k,j]                    (exact, int32)
 *     Y[i,j] = fl32(fl32(isum) * (ascale[i] wscale[j])) + (bf16(z) L2)[i,j] + bias[j]
 *   qx, ascale, z as produced by svdq_w8a8_quantize_act_lowrank_down; y, the
 *   workspace and determinism as svdq_gemm_w4a4_lowrank_up. */
int svdq_w8a8_gemm_lowrank_up(const int8_t* qx, const uint16_t* ascale, const float* z,
                              const svdq_w8a8_layer* layer, int b, void* y, int y_dtype,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace svdq_w8a8_linear needs. */
size_t svdq_w8a8_linear_workspace_size(int b, int m, int n, int rank);

/* DEVICE: the whole 8-bit layer: exactly the kernels of the two entry points
 * above, back to back on `stream` (bit-identical output).  Arguments as
 * svdq_linear. */
int svdq_w8a8_linear(const uint16_t* x, const svdq_w8a8_layer* layer, int b, void* y, int y_dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ===========================================================================
 * The NVFP4 setting ([Review] sec. 8: the 4-bit setting with group size 16
 * and FP8 scales; sec. 2.2: FP4's nonuniform grid).
 *   - FP4 E2M1 codes (values 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 = sign), two
 *     per byte in the INT4 record layout: for channels 64g..64g+63 and row
 *     (or column) r one 32-byte record, byte t = code[2t] | code[2t+1] << 4;
 *     a tensor of R rows is [m/64][R][32].
 *   - One FP8 E4M3 block scale (bias 7, largest finite 448) per 16 consecutive
 *     channels, stored as bytes [m/64][R][4] (byte j = channels 64g+16j ..).
 *   - One power-of-two fp32 tensor scale t per operand placing the block
 *     scales in E4M3's range: for a block of magnitudes amax,
 *     sb = E4M3_RNE_sat(fl32(amax / 6) / t), S = sb t, and each code is
 *     E2M1_RNE_sat(fl32(v / S)) with ties to the even code and the quotient's
 *     sign (sb = 0: codes 0).
 *   - Y = t_x t_w (X^ W^) + bf16(Z) L2 + bias, X^ and W^ the dequantized codes
 *     (code value times block scale, exact in f16), fp32 accumulation.
 * ========================================================================= */

/* A prepared NVFP4 layer on the device (caller-owned DEVICE pointers).
 *   m, n, rank   as in svdq_layer (m % 64 == 0).
 *   t_x, t_w     the activation and weight tensor scales (positive powers of two).
 *   smooth_inv, l1, l2, bias   as in svdq_layer.
 *   qw           FP4 codes of R, [m/64][n][32].
 *   wscale       E4M3 block scales, bytes [m/64][n][4]. */
typedef struct svdq_fp4_layer {
  int32_t m, n, rank;
  float t_x, t_w;
  const float* smooth_inv;
  const uint8_t* qw;
  const uint8_t* wscale;
  const uint16_t* l1;
  const uint16_t* l2;
  const uint16_t* bias;
} svdq_fp4_layer;

/* HOST: offline preparation of an NVFP4 layer: steps 2-4 of [Review]
 * Algorithm 1 exactly as svdq_prepare_weights, then R quantized per output
 * column in blocks of 16 input channels with t_w = 2^ceil(log2(max|R| / 2688)).
 * The activation tensor scale comes from the calibration statistic:
 * t_x = 2^ceil(log2(A / 2688)) with A = max_k bf16(fl32(a_k / lambda_k)), the
 * largest smoothed calibration magnitude (t_x = 1 when act_amax is NULL).
 * Outputs (HOST, caller-allocated): qw [m/64][n][32], wscale [m/64][n][4],
 * l1, l2, lambda, smooth_inv, residual (nullable) as svdq_prepare_weights,
 * t_x and t_w (one float each).  Errors as svdq_prepare_weights. */
int svdq_fp4_prepare_weights(const float* W, const float* act_amax, int m, int n, int rank, float alpha,
                             uint8_t* qw, uint8_t* wscale, uint16_t* l1, uint16_t* l2, float* lambda,
                             float* smooth_inv, float* residual, float* t_x, float* t_w);

/* Bytes of device workspace svdq_fp4_quantize_act_lowrank_down needs (as
 * svdq_act_workspace_size). */
size_t svdq_fp4_act_workspace_size(int b, int m, int rank);

/* DEVICE: fused NVFP4 activation quantization + low-rank down-projection (the
 * act-quant kernel of svdq_quantize_act_lowrank_down with the NVFP4 quantizer):
 *     x~ = bf16(fl32(x * smooth_inv)); per row and 16 channels sb, codes as
 *     above with tensor scale t_x; z = x~ L1 (fp32).
 *   Outputs: qx [m/64][b][32], ascale bytes [m/64][b][4] (any alignment), z
 *   fp32 [b][rank] (NULL iff rank == 0).  t_x a positive power of two.  Other
 *   arguments as svdq_quantize_act_lowrank_down. */
int svdq_fp4_quantize_act_lowrank_down(const uint16_t* x, int b, int m, int rank, const float* smooth_inv,
                                       const uint16_t* l1, float t_x, uint8_t* qx, uint8_t* ascale, float* z,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace svdq_fp4_gemm_lowrank_up accepts (the bound of
 * svdq_gemm_workspace_size; NVFP4 tiles are never split, so the kernels do
 * not use it). */
size_t svdq_fp4_gemm_workspace_size(int b, int n, int m);

/* DEVICE: NVFP4 GEMM + low-rank up-projection:
 *     Y = t_x t_w sum_k x^[i,k] w^[k,j] + (bf16(z) L2)[i,j] + bias[j]
 *   x^ = E2M1(qx) * E4M3(ascale block), w^ likewise (exact f16 values), fp32
 *   accumulation in a fixed order (deterministic).  y, the workspace and the
 *   remaining arguments as svdq_gemm_w4a4_lowrank_up. */
int svdq_fp4_gemm_lowrank_up(const uint8_t* qx, const uint8_t* ascale, const float* z,
                             const svdq_fp4_layer* layer, int b, void* y, int y_dtype, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Bytes of device workspace svdq_fp4_linear needs. */
size_t svdq_fp4_linear_workspace_size(int b, int m, int n, int rank);

/* DEVICE: the whole NVFP4 layer: exactly the kernels of the two entry points
 * above (bit-identical output).  Arguments as svdq_linear. */
int svdq_fp4_linear(const uint16_t* x, const svdq_fp4_layer* layer, int b, void* y, int y_dtype,
                    void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_H */
