// Offline preparation of an SVDQuant layer on the host, in fp64.
//
// [Review] = "SVDQuant: How a Small High-Precision Branch Makes 4-Bit Diffusion
// Practical" (technical review of arXiv:2411.05007v4).
//   smoothing scales           sec. 3.1, Eq.(3)-(4)
//   truncated SVD / residual   sec. 5, Eq.(10), Algorithm 1 steps 3-4
//   residual INT4 quantization sec. 2.2 Eq.(1), Algorithm 1 step 5, sec. 8
//   LoRA concatenation         sec. 7, Eq.(13)
//
// The SVD is our own: randomized subspace iteration (Halko, Martinsson & Tropp,
// SIAM Review 2011, Alg. 4.4) with twice-repeated modified Gram-Schmidt, then a
// one-sided (Hestenes) Jacobi SVD of the small projected factor.  No LAPACK.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <functional>
#include <thread>
#include <vector>

#include "internal.h"

namespace svdq {

// ---------------------------------------------------------------------------
// threading
// ---------------------------------------------------------------------------
int host_threads() {
  unsigned hc = std::thread::hardware_concurrency();
  if (hc == 0) hc = 1;
  return (int)std::min(hc, 64u);
}

// Runs fn(lo, hi) over [0, count) split into contiguous chunks, one per worker.
static void parallel_for(int64_t count, const std::function<void(int64_t, int64_t)>& fn,
                         int64_t min_chunk = 1) {
  int nt = host_threads();
  int64_t chunks = std::max<int64_t>(1, std::min<int64_t>(nt, count / std::max<int64_t>(1, min_chunk)));
  if (chunks <= 1) {
    fn(0, count);
    return;
  }
  std::vector<std::thread> th;
  th.reserve(chunks);
  for (int64_t c = 0; c < chunks; ++c) {
    int64_t lo = count * c / chunks, hi = count * (c + 1) / chunks;
    th.emplace_back([&fn, lo, hi] { fn(lo, hi); });
  }
  for (auto& t : th) t.join();
}

// ---------------------------------------------------------------------------
// scalar conversions (round to nearest, ties to even)
// ---------------------------------------------------------------------------
uint16_t f32_to_f16_sat(float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  uint32_t sign = (x >> 16) & 0x8000u;
  uint32_t ax = x & 0x7FFFFFFFu;
  if (ax > 0x7F800000u) return (uint16_t)(sign | 0x7E00u);  // NaN
  if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7BFFu);  // rounds to inf: saturate at 65504
  if (ax >= 0x38800000u) {                                     // fp16 normal range, >= 2^-14
    uint32_t mant = ax & 0x7FFFFFu;
    uint32_t h = ((((ax >> 23) - 127u + 15u)) << 10) | (mant >> 13);
    uint32_t rem = mant & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1;  // carry may bump the exponent
    return (uint16_t)(sign | h);
  }
  // fp16 subnormal (or zero): value = k * 2^-24, k = nearest-even(|f| * 2^24)
  float af;
  std::memcpy(&af, &ax, 4);
  float k = std::nearbyint(af * 16777216.0f);  // exact scaling by a power of two
  return (uint16_t)(sign | (uint32_t)k);       // k == 1024 encodes 2^-14 correctly
}

float f16_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 0x1Fu, mant = h & 0x3FFu;
  float v;
  if (e == 0) {
    v = std::ldexp((float)mant, -24);
  } else if (e == 31) {
    v = mant ? NAN : INFINITY;
  } else {
    v = std::ldexp((float)(mant | 0x400u), (int)e - 25);
  }
  uint32_t bits;
  std::memcpy(&bits, &v, 4);
  bits |= sign;
  std::memcpy(&v, &bits, 4);
  return v;
}

uint16_t f64_to_bf16(double x) {
  if (std::isnan(x)) return 0x7FC0u;
  uint16_t sign = std::signbit(x) ? 0x8000u : 0u;
  double a = std::fabs(x);
  if (a == 0.0) return sign;
  int e;
  std::frexp(a, &e);            // a in [2^(e-1), 2^e)
  int eb = std::max(e - 1, -126);
  double q = std::ldexp(1.0, eb - 7);  // bf16 spacing in this binade (8 significant bits)
  double v = std::nearbyint(a / q) * q;
  if (v > 3.3895313892515355e38) return (uint16_t)(sign | 0x7F80u);
  float vf = (float)v;          // exact: v is a bf16 value
  uint32_t b;
  std::memcpy(&b, &vf, 4);
  return (uint16_t)(sign | (b >> 16));
}

float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// ---------------------------------------------------------------------------
// smoothing, Eq.(4): lambda_k = a_k^alpha / w_k^(1-alpha); 1 when a statistic is 0
// ---------------------------------------------------------------------------
void smoothing_lambda(const float* W, const float* act_amax, int m, int n, double alpha,
                      float* lam32, float* inv32) {
  parallel_for(m, [&](int64_t lo, int64_t hi) {
    for (int64_t k = lo; k < hi; ++k) {
      double lam = 1.0;
      if (act_amax) {
        double wmax = 0.0;
        const float* row = W + k * (int64_t)n;
        for (int j = 0; j < n; ++j) wmax = std::max(wmax, std::fabs((double)row[j]));
        double a = act_amax[k];
        if (a > 0.0 && wmax > 0.0) lam = std::pow(a, alpha) / std::pow(wmax, 1.0 - alpha);
      }
      float l32 = (float)lam;
      lam32[k] = l32;
      inv32[k] = (float)(1.0 / (double)l32);
    }
  }, 64);
}

// ---------------------------------------------------------------------------
// dense helpers for the SVD (row-major fp64)
// ---------------------------------------------------------------------------
// Y (m x k) = A (m x n) * X (n x k)
static void mat_mul_ax(const double* A, int m, int n, const double* X, int k, double* Y) {
  const int JB = 256;
  parallel_for(m, [&](int64_t lo, int64_t hi) {
    const int IB = 32;
    for (int64_t i0 = lo; i0 < hi; i0 += IB) {
      int64_t i1 = std::min<int64_t>(hi, i0 + IB);
      for (int64_t i = i0; i < i1; ++i) std::fill(Y + i * k, Y + (i + 1) * k, 0.0);
      for (int j0 = 0; j0 < n; j0 += JB) {
        int j1 = std::min(n, j0 + JB);
        for (int64_t i = i0; i < i1; ++i) {
          double* y = Y + i * k;
          const double* a = A + i * (int64_t)n;
          for (int j = j0; j < j1; ++j) {
            double w = a[j];
            const double* x = X + (int64_t)j * k;
            for (int c = 0; c < k; ++c) y[c] += w * x[c];
          }
        }
      }
    }
  }, 16);
}

// Z (n x k) = A^T (n x m) * Q (m x k), A is m x n
static void mat_mul_atx(const double* A, int m, int n, const double* Q, int k, double* Z) {
  parallel_for(n, [&](int64_t lo, int64_t hi) {
    const int64_t JB = 128;
    for (int64_t j0 = lo; j0 < hi; j0 += JB) {
      int64_t j1 = std::min<int64_t>(hi, j0 + JB);
      for (int64_t j = j0; j < j1; ++j) std::fill(Z + j * k, Z + (j + 1) * k, 0.0);
      for (int i = 0; i < m; ++i) {
        const double* a = A + (int64_t)i * n;
        const double* q = Q + (int64_t)i * k;
        for (int64_t j = j0; j < j1; ++j) {
          double w = a[j];
          double* z = Z + j * k;
          for (int c = 0; c < k; ++c) z[c] += w * q[c];
        }
      }
    }
  }, 64);
}

// Orthonormalise the k columns of Y (rows x k, row-major) in place with
// modified Gram-Schmidt applied twice.  If R is given, Y_in = Q R with R upper
// triangular (k x k, row-major).
static void orthonormalize(double* Y, int64_t rows, int k, double* R) {
  std::vector<double> col(rows), qi(rows);
  if (R) std::fill(R, R + (int64_t)k * k, 0.0);
  for (int j = 0; j < k; ++j) {
    for (int64_t r = 0; r < rows; ++r) col[r] = Y[r * k + j];
    double norm0 = 0.0;
    for (int64_t r = 0; r < rows; ++r) norm0 += col[r] * col[r];
    norm0 = std::sqrt(norm0);
    for (int pass = 0; pass < 2; ++pass) {
      for (int i = 0; i < j; ++i) {
        double c = 0.0;
        for (int64_t r = 0; r < rows; ++r) c += Y[r * k + i] * col[r];
        for (int64_t r = 0; r < rows; ++r) col[r] -= c * Y[r * k + i];
        if (R) R[(int64_t)i * k + j] += c;
      }
    }
    double norm = 0.0;
    for (int64_t r = 0; r < rows; ++r) norm += col[r] * col[r];
    norm = std::sqrt(norm);
    if (!(norm > 1e-13 * norm0) || norm == 0.0) {
      // numerically dependent column: replace by a unit vector orthogonal to the
      // previous ones (keeps the basis orthonormal; R gets a zero diagonal)
      for (int64_t start = 0; start < rows; ++start) {
        std::fill(col.begin(), col.end(), 0.0);
        col[(start + j) % rows] = 1.0;
        for (int pass = 0; pass < 2; ++pass)
          for (int i = 0; i < j; ++i) {
            double c = 0.0;
            for (int64_t r = 0; r < rows; ++r) c += Y[r * k + i] * col[r];
            for (int64_t r = 0; r < rows; ++r) col[r] -= c * Y[r * k + i];
          }
        norm = 0.0;
        for (int64_t r = 0; r < rows; ++r) norm += col[r] * col[r];
        norm = std::sqrt(norm);
        if (norm > 0.5) break;
      }
      if (R) R[(int64_t)j * k + j] = 0.0;
    } else if (R) {
      R[(int64_t)j * k + j] = norm;
    }
    for (int64_t r = 0; r < rows; ++r) Y[r * k + j] = col[r] / norm;
  }
}

// One-sided Jacobi SVD of a square k x k matrix A (row-major, overwritten):
// A V = U Sigma.  On return A holds U Sigma column-wise, V the rotations.
static bool jacobi_svd(double* A, int k, double* V) {
  for (int i = 0; i < k; ++i)
    for (int j = 0; j < k; ++j) V[(int64_t)i * k + j] = (i == j) ? 1.0 : 0.0;
  const double eps = 1e-15;
  for (int sweep = 0; sweep < 80; ++sweep) {
    bool rotated = false;
    for (int p = 0; p < k - 1; ++p) {
      for (int q = p + 1; q < k; ++q) {
        double alpha = 0, beta = 0, gamma = 0;
        for (int r = 0; r < k; ++r) {
          double ap = A[(int64_t)r * k + p], aq = A[(int64_t)r * k + q];
          alpha += ap * ap;
          beta += aq * aq;
          gamma += ap * aq;
        }
        if (gamma == 0.0 || std::fabs(gamma) <= eps * std::sqrt(alpha * beta)) continue;
        rotated = true;
        double zeta = (beta - alpha) / (2.0 * gamma);
        double t = (zeta >= 0 ? 1.0 : -1.0) / (std::fabs(zeta) + std::sqrt(1.0 + zeta * zeta));
        double c = 1.0 / std::sqrt(1.0 + t * t), s = c * t;
        for (int r = 0; r < k; ++r) {
          double ap = A[(int64_t)r * k + p], aq = A[(int64_t)r * k + q];
          A[(int64_t)r * k + p] = c * ap - s * aq;
          A[(int64_t)r * k + q] = s * ap + c * aq;
          double vp = V[(int64_t)r * k + p], vq = V[(int64_t)r * k + q];
          V[(int64_t)r * k + p] = c * vp - s * vq;
          V[(int64_t)r * k + q] = s * vp + c * vq;
        }
      }
    }
    if (!rotated) return true;
  }
  return false;
}

static uint64_t splitmix64(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

bool truncated_svd(const double* Wt, int m, int n, int r, double* L1, double* L2) {
  if (r == 0) return true;
  const int mn = std::min(m, n);
  // Oversampled width and power iterations sized for flat (Marchenko-Pastur)
  // spectra, where sigma_r and sigma_{r+1} nearly coincide: the rank-r tail
  // energy comes within ~1e-5 of the optimum on such matrices.
  const int k = std::min(mn, r + std::max(32, r));
  const int power_iters = 8;

  // Gaussian test matrix Omega (n x k), Box-Muller on a fixed-seed splitmix64 stream
  std::vector<double> omega((int64_t)n * k);
  uint64_t state = 0x5EED5EEDull;
  for (int64_t i = 0; i < (int64_t)n * k; i += 2) {
    double u1 = ((splitmix64(state) >> 11) + 1) * (1.0 / 9007199254740993.0);
    double u2 = (splitmix64(state) >> 11) * (1.0 / 9007199254740992.0);
    double rad = std::sqrt(-2.0 * std::log(u1));
    omega[i] = rad * std::cos(2.0 * M_PI * u2);
    if (i + 1 < (int64_t)n * k) omega[i + 1] = rad * std::sin(2.0 * M_PI * u2);
  }
  std::vector<double> Y((int64_t)m * k), Zn((int64_t)n * k);
  mat_mul_ax(Wt, m, n, omega.data(), k, Y.data());
  orthonormalize(Y.data(), m, k, nullptr);
  for (int it = 0; it < power_iters; ++it) {
    mat_mul_atx(Wt, m, n, Y.data(), k, Zn.data());
    orthonormalize(Zn.data(), n, k, nullptr);
    mat_mul_ax(Wt, m, n, Zn.data(), k, Y.data());
    orthonormalize(Y.data(), m, k, nullptr);
  }
  // B^T = W^T Q (n x k) = Q2 R2;  R2 = U_R Sigma V_R^T  =>  W ~ (Q V_R) Sigma (Q2 U_R)^T
  mat_mul_atx(Wt, m, n, Y.data(), k, Zn.data());
  std::vector<double> R2((int64_t)k * k), VR((int64_t)k * k);
  orthonormalize(Zn.data(), n, k, R2.data());
  if (!jacobi_svd(R2.data(), k, VR.data())) return false;
  std::vector<double> sig(k);
  for (int c = 0; c < k; ++c) {
    double s = 0;
    for (int rr = 0; rr < k; ++rr) s += R2[(int64_t)rr * k + c] * R2[(int64_t)rr * k + c];
    sig[c] = std::sqrt(s);
  }
  std::vector<int> order(k);
  for (int c = 0; c < k; ++c) order[c] = c;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return sig[a] > sig[b]; });

  for (int t = 0; t < r; ++t) {
    int c = order[t];
    double s = sig[c];
    // left vector u = Q * VR[:, c]; right vector v = Q2 * (R2[:, c] / s)
    std::vector<double> u(m), v(n);
    for (int i = 0; i < m; ++i) {
      double acc = 0;
      for (int j = 0; j < k; ++j) acc += Y[(int64_t)i * k + j] * VR[(int64_t)j * k + c];
      u[i] = acc;
    }
    for (int j = 0; j < n; ++j) {
      double acc = 0;
      if (s > 0)
        for (int q = 0; q < k; ++q) acc += Zn[(int64_t)j * k + q] * (R2[(int64_t)q * k + c] / s);
      v[j] = acc;
    }
    // sign convention: the largest-magnitude entry of u is positive
    int imax = 0;
    for (int i = 1; i < m; ++i)
      if (std::fabs(u[i]) > std::fabs(u[imax])) imax = i;
    double sgn = u[imax] < 0 ? -1.0 : 1.0;
    for (int i = 0; i < m; ++i) L1[(int64_t)i * r + t] = sgn * u[i] * s;
    for (int j = 0; j < n; ++j) L2[(int64_t)t * n + j] = sgn * v[j];
  }
  return true;
}

// ---------------------------------------------------------------------------
// residual INT4 quantization: per output column j, per 64-row group g,
// s = fp16(fl32(amax / 7)), q = clamp(rint(fl32(v / s)), -7, 7), q = 0 if s == 0
// ---------------------------------------------------------------------------
void quantize_residual(const float* R, int m, int n, uint8_t* qw, uint16_t* wscale) {
  const int G = m / SVDQ_GROUP;
  parallel_for((int64_t)G * n, [&](int64_t lo, int64_t hi) {
    for (int64_t idx = lo; idx < hi; ++idx) {
      int g = (int)(idx / n), j = (int)(idx % n);
      float amax = 0.0f;
      for (int kk = 0; kk < SVDQ_GROUP; ++kk)
        amax = std::max(amax, std::fabs(R[(int64_t)(g * SVDQ_GROUP + kk) * n + j]));
      uint16_t s16 = f32_to_f16_sat(amax / 7.0f);
      float s = f16_to_f32(s16);
      wscale[(int64_t)g * n + j] = s16;
      uint8_t* rec = qw + ((int64_t)g * n + j) * 32;
      for (int t = 0; t < 32; ++t) {
        int q2[2];
        for (int h = 0; h < 2; ++h) {
          float v = R[(int64_t)(g * SVDQ_GROUP + 2 * t + h) * n + j];
          float q = 0.0f;
          if (s > 0.0f) {
            float quot = v / s;
            q = std::nearbyint(quot);
            q = std::min(7.0f, std::max(-7.0f, q));
          }
          q2[h] = (int)q;
        }
        rec[t] = (uint8_t)((q2[0] & 0xF) | ((q2[1] & 0xF) << 4));
      }
    }
  }, 256);
}

// The 8-bit setting ([Review] sec. 8): one scale per output column over all m
// rows, s = fp16(fl32(amax / 127)), codes clamp(round_even(fl32(v / s)),
// -127, 127), 0 where s = 0; 64-byte group-major records [m/64][n][64].
void quantize_residual8(const float* R, int m, int n, int8_t* qw, uint16_t* wscale) {
  constexpr int CB = 16;  // columns per task: each row is read 64 contiguous bytes at a time
  parallel_for((n + CB - 1) / CB, [&](int64_t lo, int64_t hi) {
    for (int64_t blk = lo; blk < hi; ++blk) {
      const int j0 = (int)blk * CB, j1 = std::min(n, j0 + CB);
      float amax[CB] = {};
      for (int k = 0; k < m; ++k)
        for (int j = j0; j < j1; ++j) amax[j - j0] = std::max(amax[j - j0], std::fabs(R[(int64_t)k * n + j]));
      float s[CB];
      for (int j = j0; j < j1; ++j) {
        wscale[j] = f32_to_f16_sat(amax[j - j0] / 127.0f);
        s[j - j0] = f16_to_f32(wscale[j]);
      }
      for (int k = 0; k < m; ++k)
        for (int j = j0; j < j1; ++j) {
          float q = 0.0f;
          if (s[j - j0] > 0.0f) {
            q = std::nearbyint(R[(int64_t)k * n + j] / s[j - j0]);
            q = std::min(127.0f, std::max(-127.0f, q));
          }
          qw[((int64_t)(k / SVDQ_GROUP) * n + j) * SVDQ_GROUP + k % SVDQ_GROUP] = (int8_t)q;
        }
    }
  });
}

// The NVFP4 setting ([Review] sec. 8, group 16 with FP8 scales): E4M3 block
// scales sb = E4M3_RNE_sat(fl32(amax / 6) / t), codes E2M1_RNE_sat(fl32(v / S))
// with S = sb t, ties to the even code, the quotient's sign in bit 3.
double fp4_tensor_scale(double amax) {
  if (!(amax > 0.0)) return 1.0;
  int e = 0;
  const double mnt = std::frexp(amax / (6.0 * 448.0), &e);  // q = mnt 2^e, mnt in [0.5, 1)
  return mnt == 0.5 ? std::ldexp(1.0, e - 1) : std::ldexp(1.0, e);
}

static double e4m3_round_host(double x) {  // x >= 0
  if (!(x < 448.0)) return 448.0;
  if (x == 0.0) return 0.0;
  int e = 0;
  std::frexp(x, &e);
  const int q = std::max(e - 1, -6) - 3;  // quantum exponent
  return std::min(std::nearbyint(std::ldexp(x, -q)) * std::ldexp(1.0, q), 448.0);
}

static uint8_t e4m3_bits_host(double v) {  // v a non-negative E4M3 value
  if (v == 0.0) return 0;
  int e = 0;
  const double mnt = std::frexp(v, &e);  // v = mnt 2^e
  const int ex = e - 1;
  if (ex >= -6) return (uint8_t)(((ex + 7) << 3) | (int)std::lround((mnt * 2.0 - 1.0) * 8.0));
  return (uint8_t)std::lround(std::ldexp(v, 9));
}

static uint8_t e2m1_code_host(float y) {  // RNE on the grid, saturating; ties to the even code
  const float a = std::fabs(y);
  const int idx = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return (uint8_t)(idx | (std::signbit(y) ? 8 : 0));
}

void quantize_residual_fp4(const float* R, int m, int n, double t, uint8_t* qw, uint8_t* wscale) {
  const int G = m / SVDQ_GROUP;
  parallel_for((int64_t)G * n, [&](int64_t lo, int64_t hi) {
    for (int64_t idx = lo; idx < hi; ++idx) {
      const int g = (int)(idx / n), j = (int)(idx % n);
      uint8_t* rec = qw + ((int64_t)g * n + j) * 32;
      std::memset(rec, 0, 32);
      for (int blk = 0; blk < 4; ++blk) {
        const int k0 = g * SVDQ_GROUP + 16 * blk;
        float amax = 0.0f;
        for (int kk = 0; kk < 16; ++kk) amax = std::max(amax, std::fabs(R[(int64_t)(k0 + kk) * n + j]));
        const float u = amax / 6.0f;                        // fl32(amax / 6)
        const double sb = e4m3_round_host((double)u / t);   // t a power of two: exact
        wscale[((int64_t)g * n + j) * 4 + blk] = e4m3_bits_host(sb);
        const float S = (float)(sb * t);                    // exact
        for (int kk = 0; kk < 16; ++kk) {
          const uint8_t code = S > 0.0f ? e2m1_code_host(R[(int64_t)(k0 + kk) * n + j] / S) : 0;
          const int ch = 16 * blk + kk;
          rec[ch >> 1] |= (uint8_t)(code << (4 * (ch & 1)));
        }
      }
    }
  }, 64);
}

// ---------------------------------------------------------------------------
// protected-layer candidates and their selection ([Review] sec. 5, Algorithm 1)
// ---------------------------------------------------------------------------

// R = W~ - L1 L2 with the stored bf16 factors (fp64 sums), then its INT4 codes.
static void form_residual(int m, int n, int rank, HostLayer& L) {
  std::vector<double> l2d((size_t)rank * n);
  for (size_t i = 0; i < l2d.size(); ++i) l2d[i] = bf16_to_f32(L.l2b[i]);
  L.r32.assign((size_t)m * n, 0.0f);
  parallel_for(m, [&](int64_t lo, int64_t hi) {
    std::vector<double> acc(n);
    for (int64_t i = lo; i < hi; ++i) {
      std::fill(acc.begin(), acc.end(), 0.0);
      for (int t = 0; t < rank; ++t) {
        const double a = bf16_to_f32(L.l1b[(size_t)i * rank + t]);
        const double* row = &l2d[(size_t)t * n];
        for (int j = 0; j < n; ++j) acc[j] += a * row[j];
      }
      for (int j = 0; j < n; ++j) L.r32[(size_t)i * n + j] = (float)(L.wt[(size_t)i * n + j] - acc[j]);
    }
  }, 16);
  L.qw.assign((size_t)m * n / 2, 0);
  L.wscale.assign((size_t)(m / SVDQ_GROUP) * n, 0);
  quantize_residual(L.r32.data(), m, n, L.qw.data(), L.wscale.data());
}

// bf16 factors of the rank-r SVD of A (fp64 [m][n]).
static bool factor(const double* A, int m, int n, int rank, HostLayer& L) {
  std::vector<double> L1((size_t)m * rank), L2((size_t)rank * n);
  if (rank > 0 && !truncated_svd(A, m, n, rank, L1.data(), L2.data())) return false;
  L.l1b.resize(L1.size());
  L.l2b.resize(L2.size());
  for (size_t i = 0; i < L1.size(); ++i) L.l1b[i] = f64_to_bf16(L1[i]);
  for (size_t i = 0; i < L2.size(); ++i) L.l2b[i] = f64_to_bf16(L2[i]);
  return true;
}

int build_layer(const float* W, const float* act_amax, int m, int n, int rank, double alpha, HostLayer& L) {
  L.alpha = alpha;
  L.lam32.resize(m);
  L.inv32.resize(m);
  smoothing_lambda(W, act_amax, m, n, alpha, L.lam32.data(), L.inv32.data());
  // W~ = diag(lambda) W in fp64 (Eq.(3); products of two fp32 are exact)
  L.wt.resize((size_t)m * n);
  for (int k = 0; k < m; ++k) {
    const double lk = L.lam32[k];
    for (int j = 0; j < n; ++j) L.wt[(size_t)k * n + j] = lk * (double)W[(size_t)k * n + j];
  }
  if (!factor(L.wt.data(), m, n, rank, L)) return SVDQ_ERR_NO_CONVERGENCE;
  form_residual(m, n, rank, L);
  return SVDQ_OK;
}

// INT4 code k of column j from the group-major records (two's complement nibble).
static inline int code_at(const HostLayer& L, int n, int k, int j) {
  const uint8_t byte = L.qw[((size_t)(k / SVDQ_GROUP) * n + j) * 32 + (k % SVDQ_GROUP) / 2];
  const int nib = (k & 1) ? (byte >> 4) : (byte & 0xF);
  return nib >= 8 ? nib - 16 : nib;
}

int refit_layer(int m, int n, int rank, HostLayer& L) {
  if (rank == 0) return SVDQ_OK;
  // A = W~ - Q(R) with Q(R) = s * q (exact in fp64)
  std::vector<double> A((size_t)m * n);
  parallel_for(m, [&](int64_t lo, int64_t hi) {
    for (int64_t k = lo; k < hi; ++k)
      for (int j = 0; j < n; ++j) {
        const double s = f16_to_f32(L.wscale[(size_t)(k / SVDQ_GROUP) * n + j]);
        A[(size_t)k * n + j] = L.wt[(size_t)k * n + j] - s * code_at(L, n, (int)k, j);
      }
  }, 16);
  if (!factor(A.data(), m, n, rank, L)) return SVDQ_ERR_NO_CONVERGENCE;
  form_residual(m, n, rank, L);
  return SVDQ_OK;
}

void reference_output(const float* x32, int b, const float* W, int m, int n, double* y) {
  parallel_for(b, [&](int64_t lo, int64_t hi) {
    for (int64_t i = lo; i < hi; ++i) {
      double* yr = y + (size_t)i * n;
      std::fill(yr, yr + n, 0.0);
      for (int k = 0; k < m; ++k) {
        const double xv = x32[(size_t)i * m + k];
        if (xv == 0.0) continue;
        const float* wr = W + (size_t)k * n;
        for (int j = 0; j < n; ++j) yr[j] += xv * (double)wr[j];
      }
    }
  });
}

double layer_output_sq_error(const float* x32, int b, const double* yref, int m, int n, int rank,
                             const HostLayer& L) {
  const int G = m / SVDQ_GROUP;
  // dequantized weight Q(R) = s q (exact in fp64), [m][n]
  std::vector<double> wq((size_t)m * n);
  parallel_for(m, [&](int64_t lo, int64_t hi) {
    for (int64_t k = lo; k < hi; ++k)
      for (int j = 0; j < n; ++j)
        wq[(size_t)k * n + j] = (double)f16_to_f32(L.wscale[(size_t)(k / SVDQ_GROUP) * n + j]) *
                                code_at(L, n, (int)k, j);
  }, 16);
  std::vector<double> l1d((size_t)m * rank), l2d((size_t)rank * n);
  for (size_t i = 0; i < l1d.size(); ++i) l1d[i] = bf16_to_f32(L.l1b[i]);
  for (size_t i = 0; i < l2d.size(); ++i) l2d[i] = bf16_to_f32(L.l2b[i]);
  std::vector<double> rowsq(b, 0.0);  // summed in row order below: deterministic
  parallel_for(b, [&](int64_t lo, int64_t hi) {
    std::vector<float> xt(m);
    std::vector<double> aq(m), y(n), z(rank);
    for (int64_t i = lo; i < hi; ++i) {
      double sq = 0.0;
      // x~ = bf16(fl32(x * inv32)); Q(x~) per 64-channel group (fp32 math, fp16 scale)
      for (int k = 0; k < m; ++k) {
        const float v = x32[(size_t)i * m + k] * L.inv32[k];
        xt[k] = bf16_to_f32(f64_to_bf16((double)v));
      }
      for (int g = 0; g < G; ++g) {
        float amax = 0.0f;
        for (int kk = 0; kk < SVDQ_GROUP; ++kk) amax = std::max(amax, std::fabs(xt[g * SVDQ_GROUP + kk]));
        const float s = f16_to_f32(f32_to_f16_sat(amax / 7.0f));
        for (int kk = 0; kk < SVDQ_GROUP; ++kk) {
          float q = 0.0f;
          if (s > 0.0f) q = std::min(7.0f, std::max(-7.0f, std::nearbyint(xt[g * SVDQ_GROUP + kk] / s)));
          aq[g * SVDQ_GROUP + kk] = (double)s * (double)q;
        }
      }
      // Y = Q(x~) Q(R) + bf16(x~ L1) L2
      std::fill(y.begin(), y.end(), 0.0);
      for (int k = 0; k < m; ++k) {
        if (aq[k] == 0.0) continue;
        const double* wr = &wq[(size_t)k * n];
        for (int j = 0; j < n; ++j) y[j] += aq[k] * wr[j];
      }
      for (int t = 0; t < rank; ++t) {
        double acc = 0.0;
        for (int k = 0; k < m; ++k) acc += (double)xt[k] * l1d[(size_t)k * rank + t];
        z[t] = bf16_to_f32(f64_to_bf16(acc));
      }
      for (int t = 0; t < rank; ++t) {
        const double* row = &l2d[(size_t)t * n];
        for (int j = 0; j < n; ++j) y[j] += z[t] * row[j];
      }
      for (int j = 0; j < n; ++j) {
        const double d = y[j] - yref[(size_t)i * n + j];
        sq += d * d;
      }
      rowsq[i] = sq;
    }
  });
  double total = 0.0;
  for (double v : rowsq) total += v;
  return total;
}

}  // namespace svdq
