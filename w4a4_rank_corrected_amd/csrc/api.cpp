// C-ABI entry points of the SVDQuant linear-layer library (declared in
// include/svdq.h).  Every argument is validated here, on the host, before any
// HIP call or any write to an output; then the work is handed to the host
// preparation code (prep.cpp) or the HIP kernel launchers.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "internal.h"

namespace svdq {

static thread_local char g_err[512];

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}
void clear_error() { g_err[0] = 0; }


// Plan of the act-quant kernels.  With at least 256 strips of 16 rows (b >=
// 4081), rank <= 48 and at most 3 channel groups per wave (m <= 1536), the
// wide kernel: one workgroup of 8 waves per strip, each wave over every 8th
// channel group, Z complete per workgroup (no split partials, no reduction
// launch).  With more groups per wave its two-deep ring no longer covers the
// load latency (measured slower than the split kernel and its reduction on
// the FLUX shapes, m >= 3072).  Otherwise workgroups of 64 rows and enough
// splits of the channel groups to put about 3072 waves on the chip, with at
// least 3 and at most 8 groups per split (the kernel stages 1/lambda and L1 in
// LDS act_chunk groups at a time; splits of more groups restage behind their
// own activation loads, measured 6 % slower on FLUX fc2 and the single-block
// output projection); the splits' partial Z are added in split order by a
// second kernel.  Depends only on the shape, so every setting's
// act-quant kernel, the standalone kernels and the fused layer sum Z in the
// same order.
constexpr int kActMaxSplitGroups = 8;
ActPlan act_plan(int b, int m, int rank) {
  ActPlan p;
  const int G = m / SVDQ_GROUP;
  if ((b + 15) / 16 >= 256 && act_blocks(rank) <= 3 && G <= 3 * kWideWavesPlan) {
    p.wide = 1;
    p.strips = (b + 15) / 16;
    p.splits = 1;
    p.groups_per_split = G;
    return p;
  }
  p.wide = 0;
  p.strips = (b + 63) / 64;
  int gps = G;
  if (p.strips > 0) {
    const int splits = std::max({1, (3072 + 4 * p.strips - 1) / (4 * p.strips),
                                 (G + kActMaxSplitGroups - 1) / kActMaxSplitGroups});
    gps = std::max((G + splits - 1) / splits, std::min(3, G));
  }
  p.groups_per_split = gps;
  p.splits = (G + gps - 1) / gps;
  return p;
}

}  // namespace svdq

using namespace svdq;

namespace {

constexpr size_t kAlign = 256;
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define REQUIRE(cond, code, ...)  \
  do {                            \
    if (!(cond)) {                \
      set_error(__VA_ARGS__);     \
      return (code);              \
    }                             \
  } while (0)

bool all_finite(const float* p, size_t count) {
  for (size_t i = 0; i < count; ++i)
    if (!std::isfinite(p[i])) return false;
  return true;
}

int check_group(int m, int group) {
  REQUIRE(group == SVDQ_GROUP, SVDQ_ERR_UNSUPPORTED, "group must be %d (got %d)", SVDQ_GROUP, group);
  REQUIRE(m >= SVDQ_GROUP && m % SVDQ_GROUP == 0, SVDQ_ERR_UNSUPPORTED,
          "m must be a positive multiple of %d (got %d)", SVDQ_GROUP, m);
  REQUIRE(m <= SVDQ_MAX_DIM, SVDQ_ERR_UNSUPPORTED, "m must be <= %d (got %d)", SVDQ_MAX_DIM, m);
  return SVDQ_OK;
}

// Arguments shared by the preparation entry points.
int check_prepare(const float* W, const float* act_amax, int m, int n, int rank, int group, const uint8_t* qw,
                  const uint16_t* wscale, const uint16_t* l1, const uint16_t* l2, const float* lambda,
                  const float* smooth_inv) {
  int st = check_group(m, group);
  if (st) return st;
  REQUIRE(n >= 1, SVDQ_ERR_INVALID_ARG, "n must be >= 1 (got %d)", n);
  REQUIRE(n <= SVDQ_MAX_DIM, SVDQ_ERR_UNSUPPORTED, "n must be <= %d (got %d)", SVDQ_MAX_DIM, n);
  REQUIRE(W && qw && wscale && lambda && smooth_inv, SVDQ_ERR_INVALID_ARG,
          "W, qw, wscale, lambda and smooth_inv must not be NULL");
  REQUIRE(rank >= 0 && rank <= SVDQ_MAX_RANK, SVDQ_ERR_UNSUPPORTED, "rank must be in [0, %d] (got %d)",
          SVDQ_MAX_RANK, rank);
  REQUIRE(rank <= std::min(m, n), SVDQ_ERR_INVALID_ARG, "rank %d exceeds min(m, n) = %d", rank, std::min(m, n));
  REQUIRE(rank == 0 || (l1 && l2), SVDQ_ERR_INVALID_ARG, "l1 / l2 must not be NULL when rank > 0");
  REQUIRE(all_finite(W, (size_t)m * n), SVDQ_ERR_NONFINITE, "W holds NaN or Inf");
  if (act_amax) {
    REQUIRE(all_finite(act_amax, (size_t)m), SVDQ_ERR_NONFINITE, "act_amax holds NaN or Inf");
    for (int k = 0; k < m; ++k) REQUIRE(act_amax[k] >= 0.0f, SVDQ_ERR_INVALID_ARG, "act_amax[%d] is negative", k);
  }
  return SVDQ_OK;
}

// Copy a host candidate to the caller's buffers (l1 transposed [rank][m], l2
// transposed [n][rank]).
void export_layer(const HostLayer& L, int m, int n, int rank, uint8_t* qw, uint16_t* wscale, uint16_t* l1,
                  uint16_t* l2, float* lambda, float* smooth_inv, float* residual) {
  std::memcpy(qw, L.qw.data(), L.qw.size());
  std::memcpy(wscale, L.wscale.data(), sizeof(uint16_t) * L.wscale.size());
  std::memcpy(lambda, L.lam32.data(), sizeof(float) * m);
  std::memcpy(smooth_inv, L.inv32.data(), sizeof(float) * m);
  if (rank > 0) {
    for (int i = 0; i < m; ++i)
      for (int t = 0; t < rank; ++t) l1[(size_t)t * m + i] = L.l1b[(size_t)i * rank + t];
    for (int t = 0; t < rank; ++t)
      for (int j = 0; j < n; ++j) l2[(size_t)j * rank + t] = L.l2b[(size_t)t * n + j];
  }
  if (residual) std::memcpy(residual, L.r32.data(), sizeof(float) * L.r32.size());
}

int hip_status(int err, const char* what) {
  if (err == 0) return SVDQ_OK;
  if (err == kErrKernelScratch) {
    set_error("%s: the kernel was built with register spills to scratch memory; refused", what);
    return SVDQ_ERR_UNSUPPORTED;
  }
  set_error("%s: HIP error %d (%s)", what, err, hip_error_name(err));
  return SVDQ_ERR_HIP;
}

struct LinearWorkspace {
  size_t qx_off, as_off, z_off, zpart_off, gemm_off, total;
};

// device-independent upper bound of the GEMM kernel's workspace
size_t gemm_ws_bytes(int b, int n, int m) {
  return b > 0 ? round_up(gemm_plan(b, n, m, 0).ws_bytes, kAlign) : 0;
}

LinearWorkspace linear_ws_layout(int b, int m, int n, int rank) {
  LinearWorkspace w;
  const size_t G = (size_t)(m / SVDQ_GROUP);
  ActPlan p = act_plan(b, m, rank);
  w.qx_off = 0;
  w.as_off = round_up(w.qx_off + G * (size_t)b * 32, kAlign);
  w.z_off = round_up(w.as_off + G * (size_t)b * 2, kAlign);
  w.zpart_off = round_up(w.z_off + (size_t)b * (size_t)rank * 4, kAlign);
  const size_t zpart = (rank > 0 && p.splits > 1) ? (size_t)p.splits * (size_t)b * (size_t)rank * 4 : 0;
  w.gemm_off = round_up(w.zpart_off + zpart, kAlign);
  w.total = round_up(w.gemm_off + gemm_ws_bytes(b, n, m), kAlign);
  if (b == 0) w.total = 0;
  return w;
}

int check_layer(const svdq_layer* L) {
  REQUIRE(L != nullptr, SVDQ_ERR_INVALID_ARG, "layer is NULL");
  int st = check_group(L->m, L->group);
  if (st) return st;
  REQUIRE(L->n >= 1, SVDQ_ERR_INVALID_ARG, "n must be >= 1 (got %d)", L->n);
  REQUIRE(L->n <= SVDQ_MAX_DIM, SVDQ_ERR_UNSUPPORTED, "n must be <= %d (got %d)", SVDQ_MAX_DIM, L->n);
  REQUIRE(L->rank >= 0 && L->rank <= SVDQ_MAX_RANK, SVDQ_ERR_UNSUPPORTED,
          "rank must be in [0, %d] (got %d)", SVDQ_MAX_RANK, L->rank);
  REQUIRE(L->qw && L->wscale, SVDQ_ERR_INVALID_ARG, "layer qw / wscale must not be NULL");
  REQUIRE(aligned16(L->qw), SVDQ_ERR_ALIGNMENT, "layer qw must be 16-byte aligned");
  REQUIRE(((uintptr_t)L->wscale & 1u) == 0, SVDQ_ERR_ALIGNMENT, "layer wscale must be 2-byte aligned");
  if (L->rank > 0) {
    REQUIRE(L->l2 != nullptr, SVDQ_ERR_INVALID_ARG, "layer l2 must not be NULL when rank > 0");
    REQUIRE(((uintptr_t)L->l2 & 1u) == 0, SVDQ_ERR_ALIGNMENT, "layer l2 must be 2-byte aligned");
  }
  if (L->bias) REQUIRE(((uintptr_t)L->bias & 1u) == 0, SVDQ_ERR_ALIGNMENT, "bias must be 2-byte aligned");
  return SVDQ_OK;
}

// The 8-bit layer: the checks of check_layer, with the INT8 bound on m.
int check_layer8(const svdq_w8a8_layer* L) {
  REQUIRE(L != nullptr, SVDQ_ERR_INVALID_ARG, "layer is NULL");
  int st = check_group(L->m, SVDQ_GROUP);
  if (st) return st;
  REQUIRE(L->m <= SVDQ_W8A8_MAX_M, SVDQ_ERR_UNSUPPORTED, "m must be <= %d for 8-bit codes (got %d)",
          SVDQ_W8A8_MAX_M, L->m);
  REQUIRE(L->n >= 1, SVDQ_ERR_INVALID_ARG, "n must be >= 1 (got %d)", L->n);
  REQUIRE(L->n <= SVDQ_MAX_DIM, SVDQ_ERR_UNSUPPORTED, "n must be <= %d (got %d)", SVDQ_MAX_DIM, L->n);
  REQUIRE(L->rank >= 0 && L->rank <= SVDQ_MAX_RANK, SVDQ_ERR_UNSUPPORTED,
          "rank must be in [0, %d] (got %d)", SVDQ_MAX_RANK, L->rank);
  REQUIRE(L->qw && L->wscale, SVDQ_ERR_INVALID_ARG, "layer qw / wscale must not be NULL");
  REQUIRE(aligned16(L->qw), SVDQ_ERR_ALIGNMENT, "layer qw must be 16-byte aligned");
  REQUIRE(((uintptr_t)L->wscale & 1u) == 0, SVDQ_ERR_ALIGNMENT, "layer wscale must be 2-byte aligned");
  if (L->rank > 0) {
    REQUIRE(L->l2 != nullptr, SVDQ_ERR_INVALID_ARG, "layer l2 must not be NULL when rank > 0");
    REQUIRE(((uintptr_t)L->l2 & 1u) == 0, SVDQ_ERR_ALIGNMENT, "layer l2 must be 2-byte aligned");
  }
  if (L->bias) REQUIRE(((uintptr_t)L->bias & 1u) == 0, SVDQ_ERR_ALIGNMENT, "bias must be 2-byte aligned");
  return SVDQ_OK;
}

// Workspace of the 8-bit layer: INT8 codes, per-token scales, Z, its split
// partials, the GEMM's workspace.
LinearWorkspace linear8_ws_layout(int b, int m, int n, int rank) {
  LinearWorkspace w;
  ActPlan p = act_plan(b, m, rank);
  w.qx_off = 0;
  w.as_off = round_up((size_t)m * (size_t)b, kAlign);
  w.z_off = round_up(w.as_off + (size_t)b * 2, kAlign);
  w.zpart_off = round_up(w.z_off + (size_t)b * (size_t)rank * 4, kAlign);
  const size_t zpart = (rank > 0 && p.splits > 1) ? (size_t)p.splits * (size_t)b * (size_t)rank * 4 : 0;
  w.gemm_off = round_up(w.zpart_off + zpart, kAlign);
  w.total = round_up(w.gemm_off + gemm_ws_bytes(b, n, m), kAlign);
  if (b == 0) w.total = 0;
  return w;
}

// Per-token codes, then Z = x~ L1 with the act kernel's down-projection alone
// (and the ordered split reduction).
int run_act8(const uint16_t* x, int b, int m, int rank, const float* smooth_inv, const uint16_t* l1, int8_t* qx,
             uint16_t* ascale, float* z, float* zpart, void* stream) {
  int st = hip_status(launch_act8_quant(x, b, m, smooth_inv, qx, ascale, stream), "act8_quant");
  if (st || rank == 0) return st;
  const ActPlan p = act_plan(b, m, rank);
  float* zp = p.splits > 1 ? zpart : z;
  st = hip_status(launch_act_quant_down(x, b, m, rank, smooth_inv, l1, nullptr, nullptr, zp, p, kActQuantNone, 1.0f, stream),
                  "lowrank_down");
  if (st || p.splits <= 1) return st;
  return hip_status(launch_z_reduce(zp, p.splits, b, rank, z, stream), "z_reduce");
}

// A tensor scale of the NVFP4 setting: a power of two in [2^-60, 2^60] (so
// t_x t_w stays a normal fp32 number and every scaling by it is exact).
bool fp4_scale_ok(float t) {
  if (!(t >= 0x1p-60f && t <= 0x1p60f)) return false;
  int e = 0;
  return std::frexp(t, &e) == 0.5f;
}

int check_layer_fp4(const svdq_fp4_layer* L) {
  REQUIRE(L != nullptr, SVDQ_ERR_INVALID_ARG, "layer is NULL");
  int st = check_group(L->m, SVDQ_GROUP);
  if (st) return st;
  REQUIRE(L->n >= 1, SVDQ_ERR_INVALID_ARG, "n must be >= 1 (got %d)", L->n);
  REQUIRE(L->n <= SVDQ_MAX_DIM, SVDQ_ERR_UNSUPPORTED, "n must be <= %d (got %d)", SVDQ_MAX_DIM, L->n);
  REQUIRE(L->rank >= 0 && L->rank <= SVDQ_MAX_RANK, SVDQ_ERR_UNSUPPORTED,
          "rank must be in [0, %d] (got %d)", SVDQ_MAX_RANK, L->rank);
  REQUIRE(fp4_scale_ok(L->t_x) && fp4_scale_ok(L->t_w), SVDQ_ERR_INVALID_ARG,
          "t_x and t_w must be powers of two in [2^-60, 2^60] (got %g, %g)", (double)L->t_x, (double)L->t_w);
  REQUIRE(L->qw && L->wscale, SVDQ_ERR_INVALID_ARG, "layer qw / wscale must not be NULL");
  REQUIRE(aligned16(L->qw), SVDQ_ERR_ALIGNMENT, "layer qw must be 16-byte aligned");
  REQUIRE(((uintptr_t)L->wscale & 1u) == 0, SVDQ_ERR_ALIGNMENT, "layer wscale must be 2-byte aligned");
  if (L->rank > 0) {
    REQUIRE(L->l2 != nullptr, SVDQ_ERR_INVALID_ARG, "layer l2 must not be NULL when rank > 0");
    REQUIRE(((uintptr_t)L->l2 & 1u) == 0, SVDQ_ERR_ALIGNMENT, "layer l2 must be 2-byte aligned");
  }
  if (L->bias) REQUIRE(((uintptr_t)L->bias & 1u) == 0, SVDQ_ERR_ALIGNMENT, "bias must be 2-byte aligned");
  return SVDQ_OK;
}

// Workspace of the NVFP4 layer: codes, block scales, Z, its split partials,
// the GEMM's workspace.
LinearWorkspace linear_fp4_ws_layout(int b, int m, int n, int rank) {
  LinearWorkspace w;
  const size_t G = (size_t)(m / SVDQ_GROUP);
  ActPlan p = act_plan(b, m, rank);
  w.qx_off = 0;
  w.as_off = round_up(G * (size_t)b * 32, kAlign);
  w.z_off = round_up(w.as_off + G * (size_t)b * 4, kAlign);
  w.zpart_off = round_up(w.z_off + (size_t)b * (size_t)rank * 4, kAlign);
  const size_t zpart = (rank > 0 && p.splits > 1) ? (size_t)p.splits * (size_t)b * (size_t)rank * 4 : 0;
  w.gemm_off = round_up(w.zpart_off + zpart, kAlign);
  w.total = round_up(w.gemm_off + gemm_ws_bytes(b, n, m), kAlign);
  if (b == 0) w.total = 0;
  return w;
}

// The NVFP4 act kernel, then the ordered reduction of split partial sums of Z.
int run_act_fp4(const uint16_t* x, int b, int m, int rank, const float* smooth_inv, const uint16_t* l1, float t_x,
                uint8_t* qx, uint8_t* ascale, float* z, float* zpart, void* stream) {
  const ActPlan p = act_plan(b, m, rank);
  float* zp = (rank > 0 && p.splits > 1) ? zpart : z;
  int st = hip_status(launch_act_quant_down(x, b, m, rank, smooth_inv, l1, qx, reinterpret_cast<uint16_t*>(ascale),
                                            zp, p, kActQuantFp4, t_x, stream),
                      "act_quant_lowrank_down_fp4");
  if (st || rank == 0 || p.splits <= 1) return st;
  return hip_status(launch_z_reduce(zp, p.splits, b, rank, z, stream), "z_reduce");
}

int check_y(void* y, int y_dtype, int b) {
  REQUIRE(y_dtype == SVDQ_OUT_BF16 || y_dtype == SVDQ_OUT_F32, SVDQ_ERR_INVALID_ARG,
          "y_dtype must be SVDQ_OUT_BF16 or SVDQ_OUT_F32 (got %d)", y_dtype);
  if (b > 0) {
    REQUIRE(y != nullptr, SVDQ_ERR_INVALID_ARG, "y must not be NULL");
    REQUIRE(((uintptr_t)y & (y_dtype == SVDQ_OUT_F32 ? 3u : 1u)) == 0, SVDQ_ERR_ALIGNMENT,
            "y must be element-aligned");
  }
  return SVDQ_OK;
}


}  // namespace

extern "C" {

int svdq_abi_version(void) { return 106; }

int svdq_test_set_svd_iteration_limit(int limit) { return set_eig_iteration_limit(limit); }

const char* svdq_last_error(void) { return g_err; }

const char* svdq_status_string(int status) {
  switch (status) {
    case SVDQ_OK: return "ok";
    case SVDQ_ERR_INVALID_ARG: return "invalid argument";
    case SVDQ_ERR_UNSUPPORTED: return "unsupported shape or parameter";
    case SVDQ_ERR_ALIGNMENT: return "misaligned pointer";
    case SVDQ_ERR_NONFINITE: return "non-finite input";
    case SVDQ_ERR_NO_CONVERGENCE: return "SVD did not converge";
    case SVDQ_ERR_WORKSPACE: return "workspace missing or too small";
    case SVDQ_ERR_HIP: return "HIP runtime error";
    case SVDQ_ERR_IO: return "layer file missing, unreadable or invalid";
    default: return "unknown status";
  }
}

int svdq_quantize_residual(const float* R, int m, int n, int group, uint8_t* qw, uint16_t* wscale) {
  clear_error();
  int st = check_group(m, group);
  if (st) return st;
  REQUIRE(n >= 1, SVDQ_ERR_INVALID_ARG, "n must be >= 1 (got %d)", n);
  REQUIRE(n <= SVDQ_MAX_DIM, SVDQ_ERR_UNSUPPORTED, "n must be <= %d (got %d)", SVDQ_MAX_DIM, n);
  REQUIRE(R && qw && wscale, SVDQ_ERR_INVALID_ARG, "R, qw and wscale must not be NULL");
  REQUIRE(all_finite(R, (size_t)m * n), SVDQ_ERR_NONFINITE, "R holds NaN or Inf");
  quantize_residual(R, m, n, qw, wscale);
  return SVDQ_OK;
}

int svdq_prepare_weights(const float* W, const float* act_amax, int m, int n, int rank, int group,
                         float alpha, uint8_t* qw, uint16_t* wscale, uint16_t* l1, uint16_t* l2,
                         float* lambda, float* smooth_inv, float* residual) {
  clear_error();
  int st = check_prepare(W, act_amax, m, n, rank, group, qw, wscale, l1, l2, lambda, smooth_inv);
  if (st) return st;
  REQUIRE(alpha >= 0.0f && alpha <= 1.0f, SVDQ_ERR_INVALID_ARG, "alpha must be in [0, 1] (got %g)",
          (double)alpha);
  HostLayer L;
  st = build_layer(W, act_amax, m, n, rank, (double)alpha, L);
  if (st) {
    set_error("truncated SVD did not converge (m=%d n=%d rank=%d)", m, n, rank);
    return st;
  }
  export_layer(L, m, n, rank, qw, wscale, l1, l2, lambda, smooth_inv, residual);
  return SVDQ_OK;
}

int svdq_prepare_weights_refined(const float* W, const float* act_amax, const uint16_t* x_cal, int b_cal,
                                 int m, int n, int rank, int group, const float* alphas, int n_alpha,
                                 int iters, uint8_t* qw, uint16_t* wscale, uint16_t* l1, uint16_t* l2,
                                 float* lambda, float* smooth_inv, float* residual, float* alpha_out,
                                 int* iter_out, double* rel_err_out) {
  clear_error();
  int st = check_prepare(W, act_amax, m, n, rank, group, qw, wscale, l1, l2, lambda, smooth_inv);
  if (st) return st;
  REQUIRE(x_cal != nullptr && b_cal >= 1, SVDQ_ERR_INVALID_ARG, "x_cal must hold at least one row");
  REQUIRE(b_cal <= SVDQ_MAX_DIM, SVDQ_ERR_UNSUPPORTED, "b_cal must be <= %d (got %d)", SVDQ_MAX_DIM, b_cal);
  REQUIRE(alphas != nullptr && n_alpha >= 1 && n_alpha <= 64, SVDQ_ERR_INVALID_ARG,
          "need 1 to 64 migration strengths (got %d)", n_alpha);
  for (int i = 0; i < n_alpha; ++i)
    REQUIRE(alphas[i] >= 0.0f && alphas[i] <= 1.0f, SVDQ_ERR_INVALID_ARG, "alphas[%d] = %g is outside [0, 1]", i,
            (double)alphas[i]);
  REQUIRE(iters >= 0 && iters <= 16, SVDQ_ERR_INVALID_ARG, "iters must be in [0, 16] (got %d)", iters);
  std::vector<float> x32((size_t)b_cal * m);
  for (size_t i = 0; i < x32.size(); ++i) x32[i] = bf16_to_f32(x_cal[i]);
  REQUIRE(all_finite(x32.data(), x32.size()), SVDQ_ERR_NONFINITE, "x_cal holds NaN or Inf");
  std::vector<double> yref((size_t)b_cal * n);
  reference_output(x32.data(), b_cal, W, m, n, yref.data());
  double ref_sq = 0.0;
  for (double v : yref) ref_sq += v * v;

  // every (alpha, refinement step) candidate is scored; the first best is kept
  HostLayer best;
  double best_sq = -1.0;
  int best_iter = 0;
  for (int a = 0; a < n_alpha; ++a) {
    HostLayer L;
    st = build_layer(W, act_amax, m, n, rank, (double)alphas[a], L);
    for (int it = 0; st == SVDQ_OK; ++it) {
      const double sq = layer_output_sq_error(x32.data(), b_cal, yref.data(), m, n, rank, L);
      if (best_sq < 0.0 || sq < best_sq) {
        best_sq = sq;
        best = L;
        best_iter = it;
      }
      if (it == iters || rank == 0) break;
      st = refit_layer(m, n, rank, L);
    }
    if (st) {
      set_error("truncated SVD did not converge (m=%d n=%d rank=%d)", m, n, rank);
      return st;
    }
  }
  export_layer(best, m, n, rank, qw, wscale, l1, l2, lambda, smooth_inv, residual);
  if (alpha_out) *alpha_out = (float)best.alpha;
  if (iter_out) *iter_out = best_iter;
  if (rel_err_out) *rel_err_out = ref_sq > 0.0 ? std::sqrt(best_sq / ref_sq) : std::sqrt(best_sq);
  return SVDQ_OK;
}

int svdq_append_lora(const uint16_t* l1, const uint16_t* l2, int m, int n, int rank,
                     const float* lambda, const float* A, const float* B, int k, float scale,
                     uint16_t* l1_out, uint16_t* l2_out) {
  clear_error();
  REQUIRE(m >= 1 && n >= 1, SVDQ_ERR_INVALID_ARG, "m, n must be >= 1");
  REQUIRE(m <= SVDQ_MAX_DIM && n <= SVDQ_MAX_DIM, SVDQ_ERR_UNSUPPORTED, "m, n must be <= %d", SVDQ_MAX_DIM);
  REQUIRE(k >= 1, SVDQ_ERR_INVALID_ARG, "adapter rank k must be >= 1 (got %d)", k);
  REQUIRE(rank >= 0 && rank + k <= SVDQ_MAX_RANK, SVDQ_ERR_UNSUPPORTED,
          "rank + k must be <= %d (got %d + %d)", SVDQ_MAX_RANK, rank, k);
  REQUIRE(rank == 0 || (l1 && l2), SVDQ_ERR_INVALID_ARG, "l1 / l2 must not be NULL when rank > 0");
  REQUIRE(A && B && l1_out && l2_out, SVDQ_ERR_INVALID_ARG, "A, B, l1_out, l2_out must not be NULL");
  REQUIRE(std::isfinite(scale), SVDQ_ERR_NONFINITE, "scale is not finite");
  REQUIRE(all_finite(A, (size_t)m * k) && all_finite(B, (size_t)k * n), SVDQ_ERR_NONFINITE,
          "A or B holds NaN or Inf");
  if (lambda) REQUIRE(all_finite(lambda, (size_t)m), SVDQ_ERR_NONFINITE, "lambda holds NaN or Inf");
  const int r2 = rank + k;
  // L1' = [L1 | bf16(diag(lambda) A)] stored transposed [r2][m]
  if (rank > 0) std::memmove(l1_out, l1, sizeof(uint16_t) * (size_t)rank * m);
  for (int t = 0; t < k; ++t)
    for (int i = 0; i < m; ++i) {
      double lam = lambda ? (double)lambda[i] : 1.0;
      l1_out[(size_t)(rank + t) * m + i] = f64_to_bf16(lam * (double)A[(size_t)i * k + t]);
    }
  // L2' = [L2 ; bf16(scale B)] stored transposed [n][r2]; walk rows backwards so
  // l2_out may alias l2 only if the caller wants in-place widening of a buffer
  // that already has room (not required)
  std::vector<uint16_t> row(r2);
  for (int j = 0; j < n; ++j) {
    for (int t = 0; t < rank; ++t) row[t] = l2[(size_t)j * rank + t];
    for (int t = 0; t < k; ++t) row[rank + t] = f64_to_bf16((double)scale * (double)B[(size_t)t * n + j]);
    std::memcpy(l2_out + (size_t)j * r2, row.data(), sizeof(uint16_t) * r2);
  }
  return SVDQ_OK;
}

int svdq_calibrate_act_amax(const uint16_t* x, int b, int m, float* amax, int accumulate,
                            void* stream) {
  clear_error();
  REQUIRE(b >= 0 && m >= 1, SVDQ_ERR_INVALID_ARG, "need b >= 0 and m >= 1 (got b=%d m=%d)", b, m);
  REQUIRE(b <= SVDQ_MAX_DIM && m <= SVDQ_MAX_DIM, SVDQ_ERR_UNSUPPORTED, "b and m must be <= %d", SVDQ_MAX_DIM);
  REQUIRE(m % 8 == 0, SVDQ_ERR_UNSUPPORTED, "m must be a multiple of 8 (got %d)", m);
  REQUIRE(amax != nullptr, SVDQ_ERR_INVALID_ARG, "amax must not be NULL");
  REQUIRE(((uintptr_t)amax & 3u) == 0, SVDQ_ERR_ALIGNMENT, "amax must be 4-byte aligned");
  if (b > 0) {
    REQUIRE(x != nullptr, SVDQ_ERR_INVALID_ARG, "x must not be NULL");
    REQUIRE(aligned16(x), SVDQ_ERR_ALIGNMENT, "x must be 16-byte aligned");
  }
  return hip_status(launch_calibrate(x, b, m, amax, accumulate, stream), "calibrate_act_amax");
}

// split partials of Z of the act-quant kernels (every setting plans alike)
static size_t act_ws_bytes(int b, int m, int rank) {
  if (b <= 0 || m < SVDQ_GROUP || m % SVDQ_GROUP || rank <= 0 || rank > SVDQ_MAX_RANK) return 0;
  ActPlan p = act_plan(b, m, rank);
  if (p.splits <= 1) return 0;
  return round_up((size_t)p.splits * (size_t)b * (size_t)rank * 4, kAlign);
}

size_t svdq_act_workspace_size(int b, int m, int rank) { return act_ws_bytes(b, m, rank); }

int svdq_quantize_act_lowrank_down(const uint16_t* x, int b, int m, int rank, int group,
                                   const float* smooth_inv, const uint16_t* l1, uint8_t* qx,
                                   uint16_t* ascale, float* z, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  clear_error();
  int st = check_group(m, group);
  if (st) return st;
  REQUIRE(b >= 0, SVDQ_ERR_INVALID_ARG, "b must be >= 0 (got %d)", b);
  REQUIRE(b <= SVDQ_MAX_DIM, SVDQ_ERR_UNSUPPORTED, "b must be <= %d (got %d)", SVDQ_MAX_DIM, b);
  REQUIRE(rank >= 0 && rank <= SVDQ_MAX_RANK, SVDQ_ERR_UNSUPPORTED, "rank must be in [0, %d] (got %d)",
          SVDQ_MAX_RANK, rank);
  if (b == 0) return SVDQ_OK;
  REQUIRE(x && qx && ascale, SVDQ_ERR_INVALID_ARG, "x, qx and ascale must not be NULL");
  REQUIRE(aligned16(x) && aligned16(qx), SVDQ_ERR_ALIGNMENT, "x and qx must be 16-byte aligned");
  REQUIRE(((uintptr_t)ascale & 1u) == 0, SVDQ_ERR_ALIGNMENT, "ascale must be 2-byte aligned");
  if (smooth_inv) REQUIRE(aligned16(smooth_inv), SVDQ_ERR_ALIGNMENT, "smooth_inv must be 16-byte aligned");
  if (rank > 0) {
    REQUIRE(l1 && z, SVDQ_ERR_INVALID_ARG, "l1 and z must not be NULL when rank > 0");
    REQUIRE(aligned16(l1), SVDQ_ERR_ALIGNMENT, "l1 must be 16-byte aligned");
    REQUIRE(((uintptr_t)z & 3u) == 0, SVDQ_ERR_ALIGNMENT, "z must be 4-byte aligned");
  }
  ActPlan p = act_plan(b, m, rank);
  const size_t need = svdq_act_workspace_size(b, m, rank);
  if (need > 0) {
    REQUIRE(workspace != nullptr && workspace_bytes >= need, SVDQ_ERR_WORKSPACE,
            "workspace of %zu bytes needed (got %zu)", need, workspace ? workspace_bytes : (size_t)0);
    REQUIRE(((uintptr_t)workspace & 15u) == 0, SVDQ_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  }
  float* zpart = (rank > 0 && p.splits > 1) ? (float*)workspace : z;
  st = hip_status(launch_act_quant_down(x, b, m, rank, smooth_inv, l1, qx, ascale, zpart, p, kActQuantInt4, 1.0f, stream),
                  "act_quant_lowrank_down");
  if (st) return st;
  if (rank > 0 && p.splits > 1)
    st = hip_status(launch_z_reduce(zpart, p.splits, b, rank, z, stream), "z_reduce");
  return st;
}

size_t svdq_gemm_workspace_size(int b, int n, int m) {
  if (b <= 0 || n <= 0 || m < SVDQ_GROUP || m % SVDQ_GROUP) return 0;
  return gemm_ws_bytes(b, n, m);
}

int svdq_gemm_schedule(int b, int n, int m, int setting, int* info) {
  clear_error();
  REQUIRE(info, SVDQ_ERR_INVALID_ARG, "info must not be NULL");
  REQUIRE(setting == SVDQ_GEMM_INT4 || setting == SVDQ_GEMM_W8A8 || setting == SVDQ_GEMM_FP4,
          SVDQ_ERR_INVALID_ARG, "unknown GEMM setting %d", setting);
  REQUIRE(b >= 0 && n >= 1, SVDQ_ERR_INVALID_ARG, "need b >= 0 and n >= 1 (got b=%d, n=%d)", b, n);
  REQUIRE(b <= SVDQ_MAX_DIM && n <= SVDQ_MAX_DIM, SVDQ_ERR_UNSUPPORTED, "b and n must be <= %d (got b=%d, n=%d)",
          SVDQ_MAX_DIM, b, n);
  int st = check_group(m, SVDQ_GROUP);
  if (st) return st;
  REQUIRE(setting != SVDQ_GEMM_W8A8 || m <= SVDQ_W8A8_MAX_M, SVDQ_ERR_UNSUPPORTED,
          "the 8-bit setting needs m <= %d (got %d)", SVDQ_W8A8_MAX_M, m);
  const int fmt = setting == SVDQ_GEMM_W8A8 ? kFmtInt8 : setting == SVDQ_GEMM_FP4 ? kFmtFp4 : kFmtInt4;
  const GemmPlan p = gemm_plan(b, n, m, device_cus(), fmt);
  info[0] = p.tiles_m * p.tiles_n;
  info[1] = p.grid;
  info[2] = p.split ? p.split_grid : 0;
  info[3] = p.split ? p.split_tiles : 0;
  info[4] = p.wg_per_cu;
  return SVDQ_OK;
}

int svdq_gemm_w4a4_lowrank_up(const uint8_t* qx, const uint16_t* ascale, const float* z,
                              const svdq_layer* layer, int b, void* y, int y_dtype, void* workspace,
                              size_t workspace_bytes, void* stream) {
  clear_error();
  int st = check_layer(layer);
  if (st) return st;
  REQUIRE(b >= 0, SVDQ_ERR_INVALID_ARG, "b must be >= 0 (got %d)", b);
  REQUIRE(b <= SVDQ_MAX_DIM, SVDQ_ERR_UNSUPPORTED, "b must be <= %d (got %d)", SVDQ_MAX_DIM, b);
  st = check_y(y, y_dtype, b);
  if (st) return st;
  if (b == 0) return SVDQ_OK;
  REQUIRE(qx && ascale, SVDQ_ERR_INVALID_ARG, "qx and ascale must not be NULL");
  REQUIRE(aligned16(qx), SVDQ_ERR_ALIGNMENT, "qx must be 16-byte aligned");
  REQUIRE(((uintptr_t)ascale & 1u) == 0, SVDQ_ERR_ALIGNMENT, "ascale must be 2-byte aligned");
  if (layer->rank > 0) {
    REQUIRE(z != nullptr, SVDQ_ERR_INVALID_ARG, "z must not be NULL when rank > 0");
    REQUIRE(((uintptr_t)z & 3u) == 0, SVDQ_ERR_ALIGNMENT, "z must be 4-byte aligned");
  }
  const size_t need = gemm_ws_bytes(b, layer->n, layer->m);
  if (need > 0) {
    REQUIRE(workspace != nullptr && workspace_bytes >= need, SVDQ_ERR_WORKSPACE,
            "workspace of %zu bytes needed (got %zu)", need, workspace ? workspace_bytes : (size_t)0);
    REQUIRE(((uintptr_t)workspace & 15u) == 0, SVDQ_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  }
  return hip_status(launch_gemm_up(qx, ascale, z, *layer, b, y, y_dtype, workspace, stream),
                    "gemm_w4a4_lowrank_up");
}

size_t svdq_linear_workspace_size(int b, int m, int n, int rank, int group) {
  if (group != SVDQ_GROUP || m < SVDQ_GROUP || m % SVDQ_GROUP || b <= 0 || n <= 0 || rank < 0 ||
      rank > SVDQ_MAX_RANK)
    return 0;
  return linear_ws_layout(b, m, n, rank).total;
}

// The two kernels of the layer on the workspace `ws` (laid out by
// linear_ws_layout): the act kernel (+ the ordered Z reduction when the
// channel groups are split), then the GEMM kernel.
static int run_linear(const uint16_t* x, const svdq_layer* layer, int b, void* y, int y_dtype, char* ws,
                      const LinearWorkspace& w, void* stream) {
  const int m = layer->m, rank = layer->rank;
  uint8_t* qx = (uint8_t*)(ws + w.qx_off);
  uint16_t* as = (uint16_t*)(ws + w.as_off);
  float* z = rank > 0 ? (float*)(ws + w.z_off) : nullptr;
  ActPlan p = act_plan(b, m, rank);
  float* zpart = (rank > 0 && p.splits > 1) ? (float*)(ws + w.zpart_off) : z;
  int st = hip_status(launch_act_quant_down(x, b, m, rank, layer->smooth_inv, layer->l1, qx, as, zpart, p,
                                            kActQuantInt4, 1.0f, stream),
                      "act_quant_lowrank_down");
  if (st) return st;
  if (rank > 0 && p.splits > 1) {
    st = hip_status(launch_z_reduce(zpart, p.splits, b, rank, z, stream), "z_reduce");
    if (st) return st;
  }
  return hip_status(launch_gemm_up(qx, as, z, *layer, b, y, y_dtype, ws + w.gemm_off, stream),
                    "gemm_w4a4_lowrank_up");
}

// Checks shared by svdq_linear and svdq_linear_noalloc (everything but the
// workspace).  Sets *done when there is nothing to launch (b == 0).
static int check_linear(const uint16_t* x, const svdq_layer* layer, int b, void* y, int y_dtype, bool* done) {
  *done = false;
  int st = check_layer(layer);
  if (st) return st;
  REQUIRE(b >= 0, SVDQ_ERR_INVALID_ARG, "b must be >= 0 (got %d)", b);
  REQUIRE(b <= SVDQ_MAX_DIM, SVDQ_ERR_UNSUPPORTED, "b must be <= %d (got %d)", SVDQ_MAX_DIM, b);
  st = check_y(y, y_dtype, b);
  if (st) return st;
  if (b == 0) {
    *done = true;
    return SVDQ_OK;
  }
  REQUIRE(x != nullptr, SVDQ_ERR_INVALID_ARG, "x must not be NULL");
  REQUIRE(aligned16(x), SVDQ_ERR_ALIGNMENT, "x must be 16-byte aligned");
  if (layer->smooth_inv)
    REQUIRE(aligned16(layer->smooth_inv), SVDQ_ERR_ALIGNMENT, "smooth_inv must be 16-byte aligned");
  if (layer->rank > 0) {
    REQUIRE(layer->l1 != nullptr, SVDQ_ERR_INVALID_ARG, "layer l1 must not be NULL when rank > 0");
    REQUIRE(aligned16(layer->l1), SVDQ_ERR_ALIGNMENT, "layer l1 must be 16-byte aligned");
  }
  return SVDQ_OK;
}

int svdq_linear(const uint16_t* x, const svdq_layer* layer, int b, void* y, int y_dtype,
                void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  bool done = false;
  int st = check_linear(x, layer, b, y, y_dtype, &done);
  if (st || done) return st;
  LinearWorkspace w = linear_ws_layout(b, layer->m, layer->n, layer->rank);
  REQUIRE(workspace != nullptr && workspace_bytes >= w.total, SVDQ_ERR_WORKSPACE,
          "workspace of %zu bytes needed (got %zu)", w.total, workspace ? workspace_bytes : (size_t)0);
  REQUIRE(((uintptr_t)workspace & (kAlign - 1)) == 0, SVDQ_ERR_ALIGNMENT,
          "workspace must be %zu-byte aligned", kAlign);
  return run_linear(x, layer, b, y, y_dtype, (char*)workspace, w, stream);
}

size_t svdq_linear_noalloc_max_workspace(void) { return kScratchBytes; }

int svdq_linear_noalloc(const uint16_t* x, const svdq_layer* layer, int b, void* y, int y_dtype, void* stream) {
  clear_error();
  bool done = false;
  int st = check_linear(x, layer, b, y, y_dtype, &done);
  if (st || done) return st;
  LinearWorkspace w = linear_ws_layout(b, layer->m, layer->n, layer->rank);
  REQUIRE(w.total <= kScratchBytes, SVDQ_ERR_WORKSPACE,
          "layer needs %zu bytes of workspace, above the %zu bytes of device scratch of svdq_linear_noalloc "
          "(use svdq_linear with a caller workspace)",
          w.total, kScratchBytes);
  void* scratch = nullptr;
  st = hip_status(scratch_buffer(&scratch), "device scratch lookup");
  if (st) return st;
  return run_linear(x, layer, b, y, y_dtype, (char*)scratch, w, stream);
}

size_t svdq_linear_unfused_workspace_size(int b, int m, int n, int rank, int group) {
  const size_t fused = svdq_linear_workspace_size(b, m, n, rank, group);
  if (fused == 0) return 0;
  return round_up(fused, kAlign) + (rank > 0 ? (size_t)b * (size_t)n * 4 : 0);
}

int svdq_linear_unfused(const uint16_t* x, const svdq_layer* layer, int b, void* y, int y_dtype,
                        void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  int st = check_layer(layer);
  if (st) return st;
  REQUIRE(b >= 0, SVDQ_ERR_INVALID_ARG, "b must be >= 0 (got %d)", b);
  REQUIRE(b <= SVDQ_MAX_DIM, SVDQ_ERR_UNSUPPORTED, "b must be <= %d (got %d)", SVDQ_MAX_DIM, b);
  st = check_y(y, y_dtype, b);
  if (st) return st;
  if (b == 0) return SVDQ_OK;
  const int m = layer->m, n = layer->n, rank = layer->rank;
  REQUIRE(aligned16(y), SVDQ_ERR_ALIGNMENT, "y must be 16-byte aligned");
  REQUIRE(x != nullptr, SVDQ_ERR_INVALID_ARG, "x must not be NULL");
  REQUIRE(aligned16(x), SVDQ_ERR_ALIGNMENT, "x must be 16-byte aligned");
  if (layer->smooth_inv)
    REQUIRE(aligned16(layer->smooth_inv), SVDQ_ERR_ALIGNMENT, "smooth_inv must be 16-byte aligned");
  if (rank > 0) {
    REQUIRE(layer->l1 != nullptr, SVDQ_ERR_INVALID_ARG, "layer l1 must not be NULL when rank > 0");
    REQUIRE(aligned16(layer->l1), SVDQ_ERR_ALIGNMENT, "layer l1 must be 16-byte aligned");
  }
  const LinearWorkspace w = linear_ws_layout(b, m, n, rank);
  const size_t y2_off = round_up(w.total, kAlign);
  const size_t need = svdq_linear_unfused_workspace_size(b, m, n, rank, SVDQ_GROUP);
  REQUIRE(workspace != nullptr && workspace_bytes >= need, SVDQ_ERR_WORKSPACE,
          "workspace of %zu bytes needed (got %zu)", need, workspace ? workspace_bytes : (size_t)0);
  REQUIRE(((uintptr_t)workspace & (kAlign - 1)) == 0, SVDQ_ERR_ALIGNMENT,
          "workspace must be %zu-byte aligned", kAlign);
  char* ws = (char*)workspace;
  uint8_t* qx = (uint8_t*)(ws + w.qx_off);
  uint16_t* as = (uint16_t*)(ws + w.as_off);
  // 1. activation quantization alone
  const ActPlan p0 = act_plan(b, m, 0);
  st = hip_status(launch_act_quant_down(x, b, m, 0, layer->smooth_inv, nullptr, qx, as, nullptr, p0,
                                        kActQuantInt4, 1.0f, stream),
                  "act_quant");
  if (st) return st;
  // 2. the W4A4 product (+ bias) into y
  svdq_layer M = *layer;
  M.rank = 0;
  M.l1 = nullptr;
  M.l2 = nullptr;
  st = hip_status(launch_gemm_up(qx, as, nullptr, M, b, y, y_dtype, ws + w.gemm_off, stream), "gemm_w4a4");
  if (st || rank == 0) return st;
  // 3. the down-projection alone, reading x again
  float* z = (float*)(ws + w.z_off);
  const ActPlan p = act_plan(b, m, rank);
  float* zpart = p.splits > 1 ? (float*)(ws + w.zpart_off) : z;
  st = hip_status(launch_act_quant_down(x, b, m, rank, layer->smooth_inv, layer->l1, nullptr, nullptr, zpart,
                                        p, kActQuantNone, 1.0f, stream),
                  "lowrank_down");
  if (st) return st;
  if (p.splits > 1) {
    st = hip_status(launch_z_reduce(zpart, p.splits, b, rank, z, stream), "z_reduce");
    if (st) return st;
  }
  // 4. the up-projection alone, into a second b x n tensor; 5. the addition
  st = hip_status(launch_lowrank_up(z, *layer, b, ws + y2_off, y_dtype, stream), "lowrank_up");
  if (st) return st;
  return hip_status(launch_add(y, ws + y2_off, (size_t)b * (size_t)n, y_dtype, stream), "add");
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The 8-bit setting ([Review] sec. 8)
// ---------------------------------------------------------------------------
extern "C" {

int svdq_w8a8_prepare_weights(const float* W, const float* act_amax, int m, int n, int rank, float alpha,
                              int8_t* qw, uint16_t* wscale, uint16_t* l1, uint16_t* l2, float* lambda,
                              float* smooth_inv, float* residual) {
  clear_error();
  // the INT4 buffers are not used: pass the 8-bit ones for the NULL checks
  int st = check_prepare(W, act_amax, m, n, rank, SVDQ_GROUP, reinterpret_cast<const uint8_t*>(qw), wscale, l1,
                         l2, lambda, smooth_inv);
  if (st) return st;
  REQUIRE(m <= SVDQ_W8A8_MAX_M, SVDQ_ERR_UNSUPPORTED, "m must be <= %d for 8-bit codes (got %d)",
          SVDQ_W8A8_MAX_M, m);
  REQUIRE(alpha >= 0.0f && alpha <= 1.0f, SVDQ_ERR_INVALID_ARG, "alpha must be in [0, 1] (got %g)",
          (double)alpha);
  HostLayer L;
  st = build_layer(W, act_amax, m, n, rank, (double)alpha, L);
  if (st) {
    set_error("truncated SVD did not converge (m=%d n=%d rank=%d)", m, n, rank);
    return st;
  }
  quantize_residual8(L.r32.data(), m, n, qw, wscale);
  std::memcpy(lambda, L.lam32.data(), sizeof(float) * m);
  std::memcpy(smooth_inv, L.inv32.data(), sizeof(float) * m);
  for (int i = 0; i < m && rank > 0; ++i)
    for (int t = 0; t < rank; ++t) l1[(size_t)t * m + i] = L.l1b[(size_t)i * rank + t];
  for (int t = 0; t < rank; ++t)
    for (int j = 0; j < n; ++j) l2[(size_t)j * rank + t] = L.l2b[(size_t)t * n + j];
  if (residual) std::memcpy(residual, L.r32.data(), sizeof(float) * L.r32.size());
  return SVDQ_OK;
}

size_t svdq_w8a8_act_workspace_size(int b, int m, int rank) { return act_ws_bytes(b, m, rank); }

int svdq_w8a8_quantize_act_lowrank_down(const uint16_t* x, int b, int m, int rank, const float* smooth_inv,
                                        const uint16_t* l1, int8_t* qx, uint16_t* ascale, float* z,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  int st = check_group(m, SVDQ_GROUP);
  if (st) return st;
  REQUIRE(m <= SVDQ_W8A8_MAX_M, SVDQ_ERR_UNSUPPORTED, "m must be <= %d for 8-bit codes (got %d)",
          SVDQ_W8A8_MAX_M, m);
  REQUIRE(b >= 0, SVDQ_ERR_INVALID_ARG, "b must be >= 0 (got %d)", b);
  REQUIRE(b <= SVDQ_MAX_DIM, SVDQ_ERR_UNSUPPORTED, "b must be <= %d (got %d)", SVDQ_MAX_DIM, b);
  REQUIRE(rank >= 0 && rank <= SVDQ_MAX_RANK, SVDQ_ERR_UNSUPPORTED, "rank must be in [0, %d] (got %d)",
          SVDQ_MAX_RANK, rank);
  if (b == 0) return SVDQ_OK;
  REQUIRE(x && qx && ascale, SVDQ_ERR_INVALID_ARG, "x, qx and ascale must not be NULL");
  REQUIRE(aligned16(x) && aligned16(qx), SVDQ_ERR_ALIGNMENT, "x and qx must be 16-byte aligned");
  REQUIRE(((uintptr_t)ascale & 1u) == 0, SVDQ_ERR_ALIGNMENT, "ascale must be 2-byte aligned");
  if (smooth_inv) REQUIRE(aligned16(smooth_inv), SVDQ_ERR_ALIGNMENT, "smooth_inv must be 16-byte aligned");
  if (rank > 0) {
    REQUIRE(l1 && z, SVDQ_ERR_INVALID_ARG, "l1 and z must not be NULL when rank > 0");
    REQUIRE(aligned16(l1), SVDQ_ERR_ALIGNMENT, "l1 must be 16-byte aligned");
    REQUIRE(((uintptr_t)z & 3u) == 0, SVDQ_ERR_ALIGNMENT, "z must be 4-byte aligned");
  }
  const size_t need = svdq_act_workspace_size(b, m, rank);
  if (need > 0) {
    REQUIRE(workspace != nullptr && workspace_bytes >= need, SVDQ_ERR_WORKSPACE,
            "workspace of %zu bytes needed (got %zu)", need, workspace ? workspace_bytes : (size_t)0);
    REQUIRE(((uintptr_t)workspace & 15u) == 0, SVDQ_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  }
  return run_act8(x, b, m, rank, smooth_inv, l1, qx, ascale, z, (float*)workspace, stream);
}

size_t svdq_w8a8_gemm_workspace_size(int b, int n, int m) { return svdq_gemm_workspace_size(b, n, m); }

int svdq_w8a8_gemm_lowrank_up(const int8_t* qx, const uint16_t* ascale, const float* z,
                              const svdq_w8a8_layer* layer, int b, void* y, int y_dtype, void* workspace,
                              size_t workspace_bytes, void* stream) {
  clear_error();
  int st = check_layer8(layer);
  if (st) return st;
  REQUIRE(b >= 0, SVDQ_ERR_INVALID_ARG, "b must be >= 0 (got %d)", b);
  REQUIRE(b <= SVDQ_MAX_DIM, SVDQ_ERR_UNSUPPORTED, "b must be <= %d (got %d)", SVDQ_MAX_DIM, b);
  st = check_y(y, y_dtype, b);
  if (st) return st;
  if (b == 0) return SVDQ_OK;
  REQUIRE(qx && ascale, SVDQ_ERR_INVALID_ARG, "qx and ascale must not be NULL");
  REQUIRE(aligned16(qx), SVDQ_ERR_ALIGNMENT, "qx must be 16-byte aligned");
  REQUIRE(((uintptr_t)ascale & 1u) == 0, SVDQ_ERR_ALIGNMENT, "ascale must be 2-byte aligned");
  if (layer->rank > 0) {
    REQUIRE(z != nullptr, SVDQ_ERR_INVALID_ARG, "z must not be NULL when rank > 0");
    REQUIRE(((uintptr_t)z & 3u) == 0, SVDQ_ERR_ALIGNMENT, "z must be 4-byte aligned");
  }
  const size_t need = gemm_ws_bytes(b, layer->n, layer->m);
  if (need > 0) {
    REQUIRE(workspace != nullptr && workspace_bytes >= need, SVDQ_ERR_WORKSPACE,
            "workspace of %zu bytes needed (got %zu)", need, workspace ? workspace_bytes : (size_t)0);
    REQUIRE(((uintptr_t)workspace & 15u) == 0, SVDQ_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  }
  return hip_status(launch_gemm8_up(qx, ascale, z, *layer, b, y, y_dtype, workspace, stream),
                    "gemm_w8a8_lowrank_up");
}

size_t svdq_w8a8_linear_workspace_size(int b, int m, int n, int rank) {
  if (m < SVDQ_GROUP || m % SVDQ_GROUP || m > SVDQ_W8A8_MAX_M || b <= 0 || n <= 0 || rank < 0 ||
      rank > SVDQ_MAX_RANK)
    return 0;
  return linear8_ws_layout(b, m, n, rank).total;
}

int svdq_w8a8_linear(const uint16_t* x, const svdq_w8a8_layer* layer, int b, void* y, int y_dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  int st = check_layer8(layer);
  if (st) return st;
  REQUIRE(b >= 0, SVDQ_ERR_INVALID_ARG, "b must be >= 0 (got %d)", b);
  REQUIRE(b <= SVDQ_MAX_DIM, SVDQ_ERR_UNSUPPORTED, "b must be <= %d (got %d)", SVDQ_MAX_DIM, b);
  st = check_y(y, y_dtype, b);
  if (st) return st;
  if (b == 0) return SVDQ_OK;
  const int m = layer->m, rank = layer->rank;
  REQUIRE(x != nullptr, SVDQ_ERR_INVALID_ARG, "x must not be NULL");
  REQUIRE(aligned16(x), SVDQ_ERR_ALIGNMENT, "x must be 16-byte aligned");
  if (layer->smooth_inv)
    REQUIRE(aligned16(layer->smooth_inv), SVDQ_ERR_ALIGNMENT, "smooth_inv must be 16-byte aligned");
  if (rank > 0) {
    REQUIRE(layer->l1 != nullptr, SVDQ_ERR_INVALID_ARG, "layer l1 must not be NULL when rank > 0");
    REQUIRE(aligned16(layer->l1), SVDQ_ERR_ALIGNMENT, "layer l1 must be 16-byte aligned");
  }
  const LinearWorkspace w = linear8_ws_layout(b, m, layer->n, rank);
  REQUIRE(workspace != nullptr && workspace_bytes >= w.total, SVDQ_ERR_WORKSPACE,
          "workspace of %zu bytes needed (got %zu)", w.total, workspace ? workspace_bytes : (size_t)0);
  REQUIRE(((uintptr_t)workspace & (kAlign - 1)) == 0, SVDQ_ERR_ALIGNMENT,
          "workspace must be %zu-byte aligned", kAlign);
  char* ws = (char*)workspace;
  int8_t* qx = (int8_t*)(ws + w.qx_off);
  uint16_t* as = (uint16_t*)(ws + w.as_off);
  float* z = rank > 0 ? (float*)(ws + w.z_off) : nullptr;
  st = run_act8(x, b, m, rank, layer->smooth_inv, layer->l1, qx, as, z, (float*)(ws + w.zpart_off), stream);
  if (st) return st;
  return hip_status(launch_gemm8_up(qx, as, z, *layer, b, y, y_dtype, ws + w.gemm_off, stream),
                    "gemm_w8a8_lowrank_up");
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The NVFP4 setting ([Review] sec. 8: group size 16 with FP8 scales)
// ---------------------------------------------------------------------------
extern "C" {

int svdq_fp4_prepare_weights(const float* W, const float* act_amax, int m, int n, int rank, float alpha,
                             uint8_t* qw, uint8_t* wscale, uint16_t* l1, uint16_t* l2, float* lambda,
                             float* smooth_inv, float* residual, float* t_x, float* t_w) {
  clear_error();
  int st = check_prepare(W, act_amax, m, n, rank, SVDQ_GROUP, qw, reinterpret_cast<const uint16_t*>(wscale), l1, l2,
                         lambda, smooth_inv);
  if (st) return st;
  REQUIRE(t_x && t_w, SVDQ_ERR_INVALID_ARG, "t_x and t_w must not be NULL");
  REQUIRE(alpha >= 0.0f && alpha <= 1.0f, SVDQ_ERR_INVALID_ARG, "alpha must be in [0, 1] (got %g)",
          (double)alpha);
  HostLayer L;
  st = build_layer(W, act_amax, m, n, rank, (double)alpha, L);
  if (st) {
    set_error("truncated SVD did not converge (m=%d n=%d rank=%d)", m, n, rank);
    return st;
  }
  double rmax = 0.0;
  for (float v : L.r32) rmax = std::max(rmax, (double)std::fabs(v));
  const double tw = fp4_tensor_scale(rmax);
  double tx = 1.0;
  if (act_amax) {
    // the largest smoothed calibration magnitude, bf16(fl32(a_k * (1/lambda_k)))
    double amax = 0.0;
    for (int k = 0; k < m; ++k)
      amax = std::max(amax, (double)bf16_to_f32(f64_to_bf16((double)(act_amax[k] * L.inv32[k]))));
    tx = fp4_tensor_scale(amax);
  }
  REQUIRE(fp4_scale_ok((float)tx) && fp4_scale_ok((float)tw), SVDQ_ERR_UNSUPPORTED,
          "tensor scales out of range (t_x %g, t_w %g)", tx, tw);
  quantize_residual_fp4(L.r32.data(), m, n, tw, qw, wscale);
  std::memcpy(lambda, L.lam32.data(), sizeof(float) * m);
  std::memcpy(smooth_inv, L.inv32.data(), sizeof(float) * m);
  for (int i = 0; i < m && rank > 0; ++i)
    for (int t = 0; t < rank; ++t) l1[(size_t)t * m + i] = L.l1b[(size_t)i * rank + t];
  for (int t = 0; t < rank; ++t)
    for (int j = 0; j < n; ++j) l2[(size_t)j * rank + t] = L.l2b[(size_t)t * n + j];
  if (residual) std::memcpy(residual, L.r32.data(), sizeof(float) * L.r32.size());
  *t_x = (float)tx;
  *t_w = (float)tw;
  return SVDQ_OK;
}

size_t svdq_fp4_act_workspace_size(int b, int m, int rank) { return act_ws_bytes(b, m, rank); }

int svdq_fp4_quantize_act_lowrank_down(const uint16_t* x, int b, int m, int rank, const float* smooth_inv,
                                       const uint16_t* l1, float t_x, uint8_t* qx, uint8_t* ascale, float* z,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  int st = check_group(m, SVDQ_GROUP);
  if (st) return st;
  REQUIRE(b >= 0, SVDQ_ERR_INVALID_ARG, "b must be >= 0 (got %d)", b);
  REQUIRE(b <= SVDQ_MAX_DIM, SVDQ_ERR_UNSUPPORTED, "b must be <= %d (got %d)", SVDQ_MAX_DIM, b);
  REQUIRE(rank >= 0 && rank <= SVDQ_MAX_RANK, SVDQ_ERR_UNSUPPORTED, "rank must be in [0, %d] (got %d)",
          SVDQ_MAX_RANK, rank);
  REQUIRE(fp4_scale_ok(t_x), SVDQ_ERR_INVALID_ARG, "t_x must be a power of two in [2^-60, 2^60] (got %g)",
          (double)t_x);
  if (b == 0) return SVDQ_OK;
  REQUIRE(x && qx && ascale, SVDQ_ERR_INVALID_ARG, "x, qx and ascale must not be NULL");
  REQUIRE(aligned16(x) && aligned16(qx), SVDQ_ERR_ALIGNMENT, "x and qx must be 16-byte aligned");
  if (smooth_inv) REQUIRE(aligned16(smooth_inv), SVDQ_ERR_ALIGNMENT, "smooth_inv must be 16-byte aligned");
  if (rank > 0) {
    REQUIRE(l1 && z, SVDQ_ERR_INVALID_ARG, "l1 and z must not be NULL when rank > 0");
    REQUIRE(aligned16(l1), SVDQ_ERR_ALIGNMENT, "l1 must be 16-byte aligned");
    REQUIRE(((uintptr_t)z & 3u) == 0, SVDQ_ERR_ALIGNMENT, "z must be 4-byte aligned");
  }
  const size_t need = svdq_act_workspace_size(b, m, rank);
  if (need > 0) {
    REQUIRE(workspace != nullptr && workspace_bytes >= need, SVDQ_ERR_WORKSPACE,
            "workspace of %zu bytes needed (got %zu)", need, workspace ? workspace_bytes : (size_t)0);
    REQUIRE(((uintptr_t)workspace & 15u) == 0, SVDQ_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  }
  return run_act_fp4(x, b, m, rank, smooth_inv, l1, t_x, qx, ascale, z, (float*)workspace, stream);
}

size_t svdq_fp4_gemm_workspace_size(int b, int n, int m) { return svdq_gemm_workspace_size(b, n, m); }

int svdq_fp4_gemm_lowrank_up(const uint8_t* qx, const uint8_t* ascale, const float* z,
                             const svdq_fp4_layer* layer, int b, void* y, int y_dtype, void* workspace,
                             size_t workspace_bytes, void* stream) {
  clear_error();
  int st = check_layer_fp4(layer);
  if (st) return st;
  REQUIRE(b >= 0, SVDQ_ERR_INVALID_ARG, "b must be >= 0 (got %d)", b);
  REQUIRE(b <= SVDQ_MAX_DIM, SVDQ_ERR_UNSUPPORTED, "b must be <= %d (got %d)", SVDQ_MAX_DIM, b);
  st = check_y(y, y_dtype, b);
  if (st) return st;
  if (b == 0) return SVDQ_OK;
  REQUIRE(qx && ascale, SVDQ_ERR_INVALID_ARG, "qx and ascale must not be NULL");
  REQUIRE(aligned16(qx), SVDQ_ERR_ALIGNMENT, "qx must be 16-byte aligned");
  REQUIRE(((uintptr_t)ascale & 1u) == 0, SVDQ_ERR_ALIGNMENT, "ascale must be 2-byte aligned");
  if (layer->rank > 0) {
    REQUIRE(z != nullptr, SVDQ_ERR_INVALID_ARG, "z must not be NULL when rank > 0");
    REQUIRE(((uintptr_t)z & 3u) == 0, SVDQ_ERR_ALIGNMENT, "z must be 4-byte aligned");
  }
  const size_t need = gemm_ws_bytes(b, layer->n, layer->m);
  if (need > 0) {
    REQUIRE(workspace != nullptr && workspace_bytes >= need, SVDQ_ERR_WORKSPACE,
            "workspace of %zu bytes needed (got %zu)", need, workspace ? workspace_bytes : (size_t)0);
    REQUIRE(((uintptr_t)workspace & 15u) == 0, SVDQ_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  }
  return hip_status(launch_gemm_fp4_up(qx, ascale, z, *layer, b, y, y_dtype, workspace, stream),
                    "gemm_fp4_lowrank_up");
}

size_t svdq_fp4_linear_workspace_size(int b, int m, int n, int rank) {
  if (m < SVDQ_GROUP || m % SVDQ_GROUP || b <= 0 || n <= 0 || rank < 0 || rank > SVDQ_MAX_RANK) return 0;
  return linear_fp4_ws_layout(b, m, n, rank).total;
}

int svdq_fp4_linear(const uint16_t* x, const svdq_fp4_layer* layer, int b, void* y, int y_dtype,
                    void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  int st = check_layer_fp4(layer);
  if (st) return st;
  REQUIRE(b >= 0, SVDQ_ERR_INVALID_ARG, "b must be >= 0 (got %d)", b);
  REQUIRE(b <= SVDQ_MAX_DIM, SVDQ_ERR_UNSUPPORTED, "b must be <= %d (got %d)", SVDQ_MAX_DIM, b);
  st = check_y(y, y_dtype, b);
  if (st) return st;
  if (b == 0) return SVDQ_OK;
  const int m = layer->m, rank = layer->rank;
  REQUIRE(x != nullptr, SVDQ_ERR_INVALID_ARG, "x must not be NULL");
  REQUIRE(aligned16(x), SVDQ_ERR_ALIGNMENT, "x must be 16-byte aligned");
  if (layer->smooth_inv)
    REQUIRE(aligned16(layer->smooth_inv), SVDQ_ERR_ALIGNMENT, "smooth_inv must be 16-byte aligned");
  if (rank > 0) {
    REQUIRE(layer->l1 != nullptr, SVDQ_ERR_INVALID_ARG, "layer l1 must not be NULL when rank > 0");
    REQUIRE(aligned16(layer->l1), SVDQ_ERR_ALIGNMENT, "layer l1 must be 16-byte aligned");
  }
  const LinearWorkspace w = linear_fp4_ws_layout(b, m, layer->n, rank);
  REQUIRE(workspace != nullptr && workspace_bytes >= w.total, SVDQ_ERR_WORKSPACE,
          "workspace of %zu bytes needed (got %zu)", w.total, workspace ? workspace_bytes : (size_t)0);
  REQUIRE(((uintptr_t)workspace & (kAlign - 1)) == 0, SVDQ_ERR_ALIGNMENT,
          "workspace must be %zu-byte aligned", kAlign);
  char* ws = (char*)workspace;
  uint8_t* qx = (uint8_t*)(ws + w.qx_off);
  uint8_t* as = (uint8_t*)(ws + w.as_off);
  float* z = rank > 0 ? (float*)(ws + w.z_off) : nullptr;
  st = run_act_fp4(x, b, m, rank, layer->smooth_inv, layer->l1, layer->t_x, qx, as, z, (float*)(ws + w.zpart_off),
                   stream);
  if (st) return st;
  return hip_status(launch_gemm_fp4_up(qx, as, z, *layer, b, y, y_dtype, ws + w.gemm_off, stream),
                    "gemm_fp4_lowrank_up");
}

}  // extern "C"
