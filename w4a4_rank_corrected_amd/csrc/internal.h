// Internal declarations shared by the C-ABI layer, the host preparation code and
// the HIP kernel launchers.  Not part of the public ABI (include/svdq.h is).
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "svdq.h"

namespace svdq {

// ---- per-thread error message (svdq_last_error) -------------------------------
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

// ---- scalar format conversions on the host (round to nearest, ties to even) ----
uint16_t f32_to_f16_sat(float f);   // fp16, saturated at +-65504
float f16_to_f32(uint16_t h);
uint16_t f64_to_bf16(double x);     // one rounding straight from fp64
float bf16_to_f32(uint16_t b);

// ---- host preparation (prep.cpp) ----------------------------------------------
// Smoothing scales of Eq.(4); lam32 / inv32 as fp32.  act_amax may be NULL.
void smoothing_lambda(const float* W, const float* act_amax, int m, int n, double alpha,
                      float* lam32, float* inv32);
// Rank-r truncated SVD of Wt (m x n, row-major fp64): L1 = U_r Sigma_r (m x r,
// row-major), L2 = V_r^T (r x n, row-major).  Returns false if it failed.
bool truncated_svd(const double* Wt, int m, int n, int r, double* L1, double* L2);
// QL iterations the SVD's eigen-solver may spend on one eigenvalue, and the
// test hook that changes it (limit < 0 restores the default); returns the
// previous limit.
constexpr int kEigIterationLimit = 60;
int set_eig_iteration_limit(int limit);
// INT4 group quantization of R (fp32 [m][n]) into group-major records.
void quantize_residual(const float* R, int m, int n, uint8_t* qw, uint16_t* wscale);
// INT8 quantization of each column of R (fp32 [m][n]) into 64-byte group-major
// records [m/64][n][64] and one fp16 scale per column.
void quantize_residual8(const float* R, int m, int n, int8_t* qw, uint16_t* wscale);
// NVFP4 quantization of each column of R (fp32 [m][n]) in blocks of 16 input
// channels with power-of-two tensor scale t: codes [m/64][n][32], E4M3 block
// scales [m/64][n][4].
void quantize_residual_fp4(const float* R, int m, int n, double t, uint8_t* qw, uint8_t* wscale);
// 2^ceil(log2(amax / (6 * 448))) (1 when amax is 0): the NVFP4 tensor scale.
double fp4_tensor_scale(double amax);

// One candidate protected layer on the host ([Review] Algorithm 1 steps 2-5).
struct HostLayer {
  double alpha = 0.5;
  std::vector<float> lam32, inv32;    // [m]
  std::vector<double> wt;             // W~ = diag(lambda) W, [m][n]
  std::vector<uint16_t> l1b, l2b;     // bf16 factors, L1 [m][r], L2 [r][n] (row-major)
  std::vector<float> r32;             // residual R = W~ - L1 L2, [m][n]
  std::vector<uint8_t> qw;            // INT4 codes of R, group-major [m/64][n][32]
  std::vector<uint16_t> wscale;       // fp16 scales [m/64][n]
};
// Steps 2-5 at migration strength alpha (act_amax NULL: lambda = 1).  Returns
// SVDQ_OK or SVDQ_ERR_NO_CONVERGENCE.
int build_layer(const float* W, const float* act_amax, int m, int n, int rank, double alpha, HostLayer& L);
// Steps 6-7: L1 L2 <- rank-r SVD of W~ - Q(R), then R and Q(R) again.
int refit_layer(int m, int n, int rank, HostLayer& L);
// Step 8's criterion: ||Y(X) - X W||_F^2 of the quantized layer on calibration
// rows x32 [b][m] (bf16 values), with X W given (fp64 [b][n]).
double layer_output_sq_error(const float* x32, int b, const double* yref, int m, int n, int rank,
                             const HostLayer& L);
// Y = X W in fp64 (x32 [b][m], W [m][n]).
void reference_output(const float* x32, int b, const float* W, int m, int n, double* y);
// Number of worker threads used by the preparation loops.
int host_threads();

// ---- device launch plan --------------------------------------------------------
// The act-quant kernel covers the rows in blocks of 64 (one 16-row strip per
// wave) and may split the channel groups of a block over `splits` workgroups;
// each split writes its own partial Z, summed in split order afterwards
// (deterministic).
// 16-column blocks of Z compiled for a rank (0, 1, 2, 3, 4, 8 or 16), and the
// LDS bytes one channel group takes in the act-quant kernel: 1/lambda (64 fp32)
// and 16 * blocks rows of L1 at a pitch of 72 bf16 (144 B, so the MFMA operand
// reads of 16 consecutive rows hit distinct banks).
constexpr int kActL1Pitch = 72;
constexpr int act_blocks(int rank) {
  return (rank + 15) / 16 <= 4 ? (rank + 15) / 16 : ((rank + 15) / 16 <= 8 ? 8 : 16);
}
constexpr int act_lds_group_bytes(int blocks) { return 256 + blocks * 16 * kActL1Pitch * 2; }
// Groups of activations each wave keeps in flight (a register ring), by the
// number of Z blocks: deeper for the light kernels, except two for ranks
// 17..32 (measured faster than four on the FLUX layers: a workgroup's first
// burst of activation loads delays the staging loads of the workgroups
// dispatched after it).
constexpr int act_depth(int blocks) { return blocks == 2 ? 2 : (blocks <= 4 ? 4 : (blocks == 8 ? 2 : 1)); }
// Groups staged in LDS at a time: the most (a multiple of the depth, at most
// 8) that fit in about 40 KB.
constexpr int act_chunk_fit(int blocks) {
  return 40960 / act_lds_group_bytes(blocks) < 8 ? 40960 / act_lds_group_bytes(blocks) : 8;
}
constexpr int act_chunk(int blocks) {
  return act_chunk_fit(blocks) - act_chunk_fit(blocks) % act_depth(blocks) > 0
             ? act_chunk_fit(blocks) - act_chunk_fit(blocks) % act_depth(blocks)
             : act_depth(blocks);
}

constexpr int kWideWavesPlan = 8;  // waves per workgroup of the wide act-quant kernel
struct ActPlan {
  int wide;              // 1: the wide kernel (16-row strips, waves over all groups, no splits)
  int strips;            // row blocks: ceil(b / 64), or ceil(b / 16) for the wide kernel
  int splits;            // workgroups per strip along the channel groups
  int groups_per_split;  // channel groups handled by one workgroup
};
ActPlan act_plan(int b, int m, int rank);

// ---- kernel launchers (HIP; return a hipError_t value, 0 = success) ------------
int launch_calibrate(const uint16_t* x, int b, int m, float* amax, int accumulate, void* stream);
// qmode: kActQuantNone (Z only), kActQuantInt4, kActQuantFp4 (tx: the power-of-
// two tensor scale of the FP4 block scales; unused otherwise).  For FP4, qx
// holds E2M1 codes in the INT4 record layout and ascale is read as bytes
// [m/64][b][4] (E4M3 block scales).
enum { kActQuantNone = 0, kActQuantInt4 = 1, kActQuantFp4 = 2 };
int launch_act_quant_down(const uint16_t* x, int b, int m, int rank, const float* smooth_inv,
                          const uint16_t* l1, uint8_t* qx, uint16_t* ascale, float* zpart,
                          const ActPlan& plan, int qmode, float tx, void* stream);
int launch_z_reduce(const float* zpart, int splits, int b, int rank, float* z, void* stream);
// Per-token INT8 codes and scales of the smoothed activations (one wave per row).
int launch_act8_quant(const uint16_t* x, int b, int m, const float* smooth_inv, int8_t* qx, uint16_t* ascale,
                      void* stream);
int launch_add(void* y, const void* t, size_t count, int y_dtype, void* stream);
int launch_lowrank_up(const float* z, const svdq_layer& L, int b, void* y, int y_dtype, void* stream);
// GEMM launch plan (plan.cpp): one tile per workgroup, or the last round's
// tiles split along the channel groups into pieces, one per workgroup, whose
// partial sums (in the workspace) a reduction kernel adds after the GEMM.
constexpr int kMaxCUs = 256;  // largest gfx950 part
struct GemmPlan {
  int tiles_m, tiles_n, G;
  int grid;             // workgroups launched
  int split;            // 1 = some tiles are split into pieces (split-K)
  int split_tiles;      // split tiles (linear tiles [0, split_tiles))
  int pieces;           // pieces per split tile
  int split_grid;       // split workgroups, split_tiles * pieces (dispatched first)
  int wg_per_cu;        // resident workgroups per CU of the kernel planned for
  int tile_n;           // output columns per tile: kGemmTileN, or kGemmTileNNarrow (INT4, few rows)
  size_t partial_bytes; // partial-sum area at the start of the workspace
  size_t ws_bytes;      // workspace bound for the shape (0 when m has too few groups to split)
};
// Operand formats of the GEMM kernel body (INT4 codes, the 8-bit setting, the
// NVFP4 setting); each has its own resident workgroups per CU.
enum GemmFormat { kFmtInt4 = 0, kFmtInt8 = 1, kFmtFp4 = 2 };
// Output tile of every GEMM build, and the resident workgroups per CU of each
// format's kernel (the same with and without split tiles).
constexpr int kGemmTileM = 128, kGemmTileN = 128;
// INT4 tiles for few rows (the wide tiles would not fill one round of slots)
constexpr int kGemmTileNNarrow = 64;
constexpr int kGemmWgPerCu[3] = {3, 3, 3};
// Split-K: pieces per split tile when full rounds of whole tiles run too
// (kMinPieces .. kMaxPieces) and when every tile is split (2 ..
// kMaxPiecesAll); each piece has at least kMinPieceGroups channel groups.
constexpr int kMinPieces = 3, kMaxPieces = 8, kMaxPiecesAll = 16, kMinPieceGroups = 8;
// The low-rank product's cost in groups: the piece that computes it (the last
// of its tile) gets this many groups fewer, so a tile's pieces end together.
constexpr int kLowRankPieceGroups = 4;
static_assert((kMaxPiecesAll - 1) * kLowRankPieceGroups < kMaxPiecesAll * (kMinPieceGroups - 1),
              "the last piece keeps at least one group");
// cus <= 0 gives the device-independent upper bound used to size workspaces
// (valid for every format); fmt selects the kernel whose residency is planned.
GemmPlan gemm_plan(int b, int n, int m, int cus, int fmt = kFmtInt4);
int device_cus();
int launch_gemm_up(const uint8_t* qx, const uint16_t* ascale, const float* z, const svdq_layer& L,
                   int b, void* y, int y_dtype, void* ws, void* stream);
int launch_gemm8_up(const int8_t* qx, const uint16_t* ascale, const float* z, const svdq_w8a8_layer& L,
                    int b, void* y, int y_dtype, void* ws, void* stream);
int launch_gemm_fp4_up(const uint8_t* qx, const uint8_t* ascale, const float* z, const svdq_fp4_layer& L, int b,
                       void* y, int y_dtype, void* ws, void* stream);
const char* hip_error_name(int err);
// Launcher status (not a hipError_t) of a kernel that would use scratch memory.
constexpr int kErrKernelScratch = -1000;

// Device scratch of the allocation-free entry point (scratch.hip): the
// current device's copy of a file-scope device array of kScratchBytes, its
// address looked up once per device.  Returns a hipError_t value (0 = success).
constexpr size_t kScratchBytes = (size_t)128 << 20;
int scratch_buffer(void** out);

}  // namespace svdq
