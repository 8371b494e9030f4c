// Offline preparation of an SVDQuant layer on the host, in fp64.
//
// [Review] = "SVDQuant: How a Small High-Precision Branch Makes 4-Bit Diffusion
// Practical" (technical review of arXiv:2411.05007v4).
//   smoothing scales           sec. 3.1, Eq.(3)-(4)
//   truncated SVD / residual   sec. 5, Eq.(10), Algorithm 1 steps 3-4
//   residual INT4 quantization sec. 2.2 Eq.(1), Algorithm 1 step 5, sec. 8
//   LoRA concatenation         sec. 7, Eq.(13)
//
// The SVD is our own: a randomized block Krylov method (Musco & Musco, NeurIPS
// 2015) with block Gram-Schmidt orthonormalisation, and a Rayleigh-Ritz step
// solved by Householder tridiagonalisation and implicit QL iterations (Golub &
// Van Loan, sec. 8.3).  No LAPACK.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <functional>
#include <limits>
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
// The inner loops are compiled twice (AVX2 and baseline x86-64) and picked at
// load time.  Every element is a plain sum of products in a fixed order
// (fp-contract off), so both clones give identical bits.
__attribute__((target_clones("avx2", "default")))
static void ax_rows(const double* A, int64_t lo, int64_t hi, int n, const double* X, int k, double* Y) {
  const int JB = 256, IB = 32;
  for (int64_t i0 = lo; i0 < hi; i0 += IB) {
    const int64_t i1 = std::min<int64_t>(hi, i0 + IB);
    for (int64_t i = i0; i < i1; ++i) std::fill(Y + i * k, Y + (i + 1) * k, 0.0);
    for (int j0 = 0; j0 < n; j0 += JB) {
      const int j1 = std::min(n, j0 + JB);
      for (int64_t i = i0; i < i1; ++i) {
        double* __restrict__ y = Y + i * k;
        const double* a = A + i * (int64_t)n;
        for (int j = j0; j < j1; ++j) {
          const double w = a[j];
          const double* __restrict__ x = X + (int64_t)j * k;
          for (int c = 0; c < k; ++c) y[c] += w * x[c];
        }
      }
    }
  }
}

__attribute__((target_clones("avx2", "default")))
static void atx_rows(const double* A, int m, int n, int64_t lo, int64_t hi, const double* Q, int k, double* Z) {
  const int64_t JB = 128;
  for (int64_t j0 = lo; j0 < hi; j0 += JB) {
    const int64_t j1 = std::min<int64_t>(hi, j0 + JB);
    for (int64_t j = j0; j < j1; ++j) std::fill(Z + j * k, Z + (j + 1) * k, 0.0);
    for (int i = 0; i < m; ++i) {
      const double* a = A + (int64_t)i * n;
      const double* __restrict__ q = Q + (int64_t)i * k;
      for (int64_t j = j0; j < j1; ++j) {
        const double w = a[j];
        double* __restrict__ z = Z + j * k;
        for (int c = 0; c < k; ++c) z[c] += w * q[c];
      }
    }
  }
}

// Y (m x k) = A (m x n) * X (n x k)
static void mat_mul_ax(const double* A, int m, int n, const double* X, int k, double* Y) {
  parallel_for(m, [&](int64_t lo, int64_t hi) { ax_rows(A, lo, hi, n, X, k, Y); }, 16);
}

// Z (n x k) = A^T (n x m) * Q (m x k), A is m x n
static void mat_mul_atx(const double* A, int m, int n, const double* Q, int k, double* Z) {
  parallel_for(n, [&](int64_t lo, int64_t hi) { atx_rows(A, m, n, lo, hi, Q, k, Z); }, 64);
}

// The operator whose singular subspace is sought, seen from its SHORT side:
// S (ls x ll) is W~ itself when m <= n, or W~^T when m > n, so every basis the
// Krylov method builds has the short length ls.
struct ShortSide {
  const double* W;  // W~, m x n row-major
  int m, n;
  bool wide() const { return m <= n; }
  int ls() const { return wide() ? m : n; }
  int ll() const { return wide() ? n : m; }
  // Y (ls x k) = S X, X is ll x k
  void apply(const double* X, int k, double* Y) const {
    if (wide()) mat_mul_ax(W, m, n, X, k, Y);
    else mat_mul_atx(W, m, n, X, k, Y);
  }
  // Z (ll x k) = S^T Y, Y is ls x k
  void apply_t(const double* Y, int k, double* Z) const {
    if (wide()) mat_mul_atx(W, m, n, Y, k, Z);
    else mat_mul_ax(W, m, n, Y, k, Z);
  }
};

// Modified Gram-Schmidt, applied twice, on the columns [c0, c1) of the
// column-major block B (each column `rows` long), among themselves; columns
// [0, c0) are already orthonormal and orthogonal to them.  A column that is
// numerically dependent (norm below 1e-12 of its norm before the projections)
// is replaced by a unit vector made orthogonal to every previous column, so
// the result is always an orthonormal set.
static void mgs_columns(double* B, int64_t rows, int c0, int c1) {
  auto proj_out = [&](double* col, int from, int upto) {
    for (int pass = 0; pass < 2; ++pass)
      for (int i = from; i < upto; ++i) {
        const double* q = B + (int64_t)i * rows;
        double c = 0.0;
        for (int64_t r = 0; r < rows; ++r) c += q[r] * col[r];
        for (int64_t r = 0; r < rows; ++r) col[r] -= c * q[r];
      }
  };
  auto norm = [&](const double* col) {
    double s = 0.0;
    for (int64_t r = 0; r < rows; ++r) s += col[r] * col[r];
    return std::sqrt(s);
  };
  for (int j = c0; j < c1; ++j) {
    double* col = B + (int64_t)j * rows;
    const double n0 = norm(col);
    proj_out(col, c0, j);
    double nr = norm(col);
    if (!(nr > 1e-12 * n0) || nr == 0.0) {
      for (int64_t start = 0; start < rows; ++start) {
        std::fill(col, col + rows, 0.0);
        col[(start + j) % rows] = 1.0;
        proj_out(col, 0, j);
        nr = norm(col);
        if (nr > 0.5) break;
      }
    }
    for (int64_t r = 0; r < rows; ++r) col[r] /= nr;
  }
}

// Orthonormalise the columns [c0, k) of Y (rows x k, row-major) against its
// (already orthonormal) columns [0, c0) and among themselves.  Blocks of
// columns are first projected against everything before them twice (block
// classical Gram-Schmidt: two passes of a product with the previous columns,
// parallel over rows, deterministic), then finished by mgs_columns on a
// column-major copy.
static void orthonormalize(double* Y, int64_t rows, int k, int c0 = 0) {
  const int BS = 32;
  for (int b0 = c0; b0 < k; b0 += BS) {
    const int b1 = std::min(k, b0 + BS), bw = b1 - b0;
    if (b0 > 0) {
      for (int pass = 0; pass < 2; ++pass) {
        // C (b0 x bw) = Y[:, :b0]^T Y[:, b0:b1], summed over row chunks in a fixed order
        const int64_t chunks = std::max<int64_t>(1, std::min<int64_t>(host_threads(), rows / 256));
        std::vector<double> part((size_t)chunks * b0 * bw, 0.0);
        parallel_for(chunks, [&](int64_t lo, int64_t hi) {
          for (int64_t ch = lo; ch < hi; ++ch) {
            double* C = &part[(size_t)ch * b0 * bw];
            const int64_t r0 = rows * ch / chunks, r1 = rows * (ch + 1) / chunks;
            for (int64_t r = r0; r < r1; ++r) {
              const double* y = Y + r * k;
              for (int i = 0; i < b0; ++i) {
                const double yi = y[i];
                double* Ci = C + (size_t)i * bw;
                for (int j = 0; j < bw; ++j) Ci[j] += yi * y[b0 + j];
              }
            }
          }
        });
        std::vector<double> C((size_t)b0 * bw, 0.0);
        for (int64_t ch = 0; ch < chunks; ++ch)
          for (size_t t = 0; t < C.size(); ++t) C[t] += part[(size_t)ch * b0 * bw + t];
        // Y[:, b0:b1] -= Y[:, :b0] C
        parallel_for(rows, [&](int64_t lo, int64_t hi) {
          double acc[BS];
          for (int64_t r = lo; r < hi; ++r) {
            double* y = Y + r * k;
            std::fill(acc, acc + bw, 0.0);
            for (int i = 0; i < b0; ++i) {
              const double yi = y[i];
              const double* Ci = &C[(size_t)i * bw];
              for (int j = 0; j < bw; ++j) acc[j] += yi * Ci[j];
            }
            for (int j = 0; j < bw; ++j) y[b0 + j] -= acc[j];
          }
        }, 64);
      }
    }
    // finish the block with MGS on a column-major copy (columns [0, b1) so that
    // dependent columns can be completed against everything before them)
    std::vector<double> cm((size_t)b1 * rows);
    for (int64_t r = 0; r < rows; ++r)
      for (int j = 0; j < b1; ++j) cm[(size_t)j * rows + r] = Y[r * k + j];
    mgs_columns(cm.data(), rows, b0, b1);
    for (int64_t r = 0; r < rows; ++r)
      for (int j = b0; j < b1; ++j) Y[r * k + j] = cm[(size_t)j * rows + r];
  }
}

// Eigen-decomposition of a symmetric K x K matrix A (row-major, full storage):
// Householder reduction to tridiagonal form with the reflections accumulated,
// then implicit QL iterations with Wilkinson-type shifts (Golub & Van Loan,
// Matrix Computations, sec. 8.3).  On return w holds the eigenvalues in
// descending order and V (K x K, row-major) the matching eigenvectors as
// columns.  Returns false if an eigenvalue needed more than the iteration
// limit (kEigIterationLimit unless a test lowered it).
// Iterations the QL phase may spend on one eigenvalue (a test hook lowers it).
static std::atomic<int> g_eig_iteration_limit{kEigIterationLimit};

int set_eig_iteration_limit(int limit) {
  return g_eig_iteration_limit.exchange(limit < 0 ? kEigIterationLimit : limit);
}

static bool sym_eig(std::vector<double>& A, int K, std::vector<double>& w, std::vector<double>& V) {
  const int iteration_limit = g_eig_iteration_limit.load();
  std::vector<double> d(K), e(K, 0.0);
  // ---- tridiagonalisation: A <- H A H for reflections H = I - beta v v^T that
  // zero column k below the subdiagonal; v is kept in A[k+1.., k]
  std::vector<double> beta(K, 0.0), p(K), q(K), v(K);
  for (int k = 0; k + 2 < K; ++k) {
    const int s = k + 1, len = K - s;
    double xn = 0.0;
    for (int i = s; i < K; ++i) xn += A[(size_t)i * K + k] * A[(size_t)i * K + k];
    xn = std::sqrt(xn);
    if (xn == 0.0) { beta[k] = 0.0; continue; }
    const double x0 = A[(size_t)s * K + k];
    const double alpha = x0 >= 0 ? -xn : xn;  // H x = alpha e_1, no cancellation in v_0
    const double v0 = x0 - alpha;
    // v = x - alpha e_1 scaled so that v_0 = 1; beta = 2 / (v^T v)
    double vv = 1.0;
    A[(size_t)s * K + k] = 1.0;
    for (int i = s + 1; i < K; ++i) {
      A[(size_t)i * K + k] /= v0;
      vv += A[(size_t)i * K + k] * A[(size_t)i * K + k];
    }
    const double bt = 2.0 / vv;
    beta[k] = bt;
    for (int i = s; i < K; ++i) v[i] = A[(size_t)i * K + k];
    // p = beta * A22 v (A22 = trailing block, symmetric, full storage)
    auto pv = [&](int64_t lo, int64_t hi) {
      for (int64_t i = s + lo; i < s + hi; ++i) {
        const double* row = &A[(size_t)i * K];
        double acc = 0.0;
        for (int j = s; j < K; ++j) acc += row[j] * v[j];
        p[i] = bt * acc;
      }
    };
    if (len >= 256) parallel_for(len, pv, 32); else pv(0, len);
    double pv_dot = 0.0;
    for (int i = s; i < K; ++i) pv_dot += p[i] * v[i];
    const double h = 0.5 * bt * pv_dot;
    for (int i = s; i < K; ++i) q[i] = p[i] - h * v[i];
    // A22 <- A22 - v q^T - q v^T
    auto upd = [&](int64_t lo, int64_t hi) {
      for (int64_t i = s + lo; i < s + hi; ++i) {
        double* row = &A[(size_t)i * K];
        const double vi = v[i], qi = q[i];
        for (int j = s; j < K; ++j) row[j] -= vi * q[j] + qi * v[j];
      }
    };
    if (len >= 256) parallel_for(len, upd, 32); else upd(0, len);
    e[k] = alpha;  // T[k+1][k]
  }
  for (int i = 0; i < K; ++i) d[i] = A[(size_t)i * K + i];
  if (K >= 2) e[K - 2] = A[(size_t)(K - 1) * K + (K - 2)];
  // Q = H_0 H_1 ... H_{K-3}, built backwards into V (row-major)
  V.assign((size_t)K * K, 0.0);
  for (int i = 0; i < K; ++i) V[(size_t)i * K + i] = 1.0;
  for (int k = K - 3; k >= 0; --k) {
    if (beta[k] == 0.0) continue;
    const int s = k + 1;
    // V[s:, s:] <- (I - beta v v^T) V[s:, s:]
    std::vector<double> t(K, 0.0);
    for (int i = s; i < K; ++i) {
      const double vi = A[(size_t)i * K + k];
      const double* row = &V[(size_t)i * K];
      for (int j = s; j < K; ++j) t[j] += vi * row[j];
    }
    for (int i = s; i < K; ++i) {
      const double f = beta[k] * A[(size_t)i * K + k];
      double* row = &V[(size_t)i * K];
      for (int j = s; j < K; ++j) row[j] -= f * t[j];
    }
  }
  // ---- implicit QL on the tridiagonal (d, e), e[i] coupling i and i+1.  The
  // rotations act on columns of V; they are applied to its transpose Vt (rows
  // contiguous), in parallel over the components.
  std::vector<double> Vt((size_t)K * K);
  for (int i = 0; i < K; ++i)
    for (int j = 0; j < K; ++j) Vt[(size_t)j * K + i] = V[(size_t)i * K + j];
  std::vector<double> cs(K), sn(K);
  for (int l = 0; l < K; ++l) {
    int iter = 0;
    for (;;) {
      int mm = l;
      for (; mm + 1 < K; ++mm) {
        const double dd = std::fabs(d[mm]) + std::fabs(d[mm + 1]);
        if (std::fabs(e[mm]) <= std::numeric_limits<double>::epsilon() * dd) break;
      }
      if (mm == l) break;
      if (++iter > iteration_limit) return false;
      // shift from the leading 2 x 2 block: its eigenvalue nearer d[l]
      double g = (d[l + 1] - d[l]) / (2.0 * e[l]);
      double r = std::hypot(g, 1.0);
      g = d[mm] - d[l] + e[l] / (g + (g >= 0 ? r : -r));
      double s = 1.0, c = 1.0, pp = 0.0;
      int i = mm - 1, stop = l - 1;
      for (; i >= l; --i) {
        const double f = s * e[i], bb = c * e[i];
        r = std::hypot(f, g);
        e[i + 1] = r;
        if (r == 0.0) {  // split: the rest of the chase is not needed
          d[i + 1] -= pp;
          e[mm] = 0.0;
          stop = i;
          break;
        }
        s = f / r;
        c = g / r;
        g = d[i + 1] - pp;
        r = (d[i] - g) * s + 2.0 * c * bb;
        pp = s * r;
        d[i + 1] = g + pp;
        g = c * r - bb;
        cs[i] = c;
        sn[i] = s;
      }
      // apply the rotations i = mm-1 .. stop+1 (in that order) to rows i, i+1 of Vt
      const int first = mm - 1, last = stop + 1;
      auto rot = [&](int64_t lo, int64_t hi) {
        for (int ii = first; ii >= last; --ii) {
          double* a = &Vt[(size_t)ii * K];
          double* b = &Vt[(size_t)(ii + 1) * K];
          const double c2 = cs[ii], s2 = sn[ii];
          for (int64_t j = lo; j < hi; ++j) {
            const double f = b[j];
            b[j] = s2 * a[j] + c2 * f;
            a[j] = c2 * a[j] - s2 * f;
          }
        }
      };
      if ((int64_t)(first - last + 1) * K >= (1 << 16)) parallel_for(K, rot, 64); else rot(0, K);
      if (stop >= l) continue;  // split: iterate again on the same l
      d[l] -= pp;
      e[l] = g;
      e[mm] = 0.0;
    }
  }
  // sort descending; eigenvector j of the result = row order[j] of Vt
  std::vector<int> order(K);
  for (int i = 0; i < K; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return d[a] > d[b]; });
  w.resize(K);
  for (int j = 0; j < K; ++j) {
    w[j] = d[order[j]];
    const double* src = &Vt[(size_t)order[j] * K];
    for (int i = 0; i < K; ++i) V[(size_t)i * K + j] = src[i];
  }
  return true;
}

static uint64_t splitmix64(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Rank-r truncated SVD by a randomized block Krylov method (Musco & Musco,
// "Randomized Block Krylov Methods for Stronger and Faster Approximate
// Singular Value Decomposition", NeurIPS 2015): a Gaussian block of width bw
// is pushed through q rounds of S S^T, the blocks of all rounds together span
// a Krylov space of dimension K = (q + 1) bw on the short side, and the
// rank-r approximation is taken from the Rayleigh-Ritz problem on that space
// (the eigen-decomposition of the K x K matrix Q^T S S^T Q).  Flat
// (Marchenko-Pastur-like) spectra, where sigma_r and sigma_{r+1} nearly
// coincide, are where plain subspace iteration converges slowly; the Krylov
// space reaches near-optimal tail energy on them at a comparable cost.  When
// K would reach the short dimension, the space is all of it and the result is
// the exact truncated SVD.
bool truncated_svd(const double* Wt, int m, int n, int r, double* L1, double* L2) {
  if (r == 0) return true;
  const ShortSide S{Wt, m, n};
  const int ls = S.ls(), ll = S.ll();
  const int bw = r + std::max(16, r / 2);
  const int kmax = std::max(480, 3 * bw);
  const int q = std::max(2, std::min(8, kmax / bw - 1));
  int K = (q + 1) * bw;
  const bool full = K >= ls;
  std::vector<double> Q;  // ls x K, orthonormal columns
  if (full) {
    K = ls;
    Q.assign((size_t)ls * K, 0.0);
    for (int i = 0; i < ls; ++i) Q[(size_t)i * K + i] = 1.0;
  } else {
    // Gaussian block Omega (ll x bw): Box-Muller on a fixed-seed splitmix64 stream
    std::vector<double> omega((size_t)ll * bw);
    uint64_t state = 0x5EED5EEDull;
    for (size_t i = 0; i < omega.size(); i += 2) {
      const double u1 = ((splitmix64(state) >> 11) + 1) * (1.0 / 9007199254740993.0);
      const double u2 = (splitmix64(state) >> 11) * (1.0 / 9007199254740992.0);
      const double rad = std::sqrt(-2.0 * std::log(u1));
      omega[i] = rad * std::cos(2.0 * M_PI * u2);
      if (i + 1 < omega.size()) omega[i + 1] = rad * std::sin(2.0 * M_PI * u2);
    }
    std::vector<double> Y((size_t)ls * bw), Z((size_t)ll * bw);
    Q.assign((size_t)ls * K, 0.0);
    S.apply(omega.data(), bw, Y.data());
    for (int it = 0;; ++it) {
      orthonormalize(Y.data(), ls, bw);
      for (int i = 0; i < ls; ++i)
        std::copy(&Y[(size_t)i * bw], &Y[(size_t)i * bw] + bw, &Q[(size_t)i * K + (size_t)it * bw]);
      if (it == q) break;
      S.apply_t(Y.data(), bw, Z.data());
      orthonormalize(Z.data(), ll, bw);
      S.apply(Z.data(), bw, Y.data());
    }
    // one orthonormal basis of the whole Krylov space (each block already is one)
    orthonormalize(Q.data(), ls, K, bw);
  }
  // P = S^T Q (ll x K); Rayleigh-Ritz on G = P^T P = Q^T S S^T Q
  std::vector<double> P((size_t)ll * K), G((size_t)K * K);
  S.apply_t(Q.data(), K, P.data());
  mat_mul_atx(P.data(), ll, K, P.data(), K, G.data());
  for (int i = 0; i < K; ++i)  // exact symmetry (both triangles are the same sums)
    for (int j = i + 1; j < K; ++j) G[(size_t)j * K + i] = G[(size_t)i * K + j];
  std::vector<double> lam, V;
  if (!sym_eig(G, K, lam, V)) return false;
  // short-side singular vectors Us = Q V_r (ls x r); long side S^T Us = P V_r
  std::vector<double> Us((size_t)ls * r, 0.0), Ul((size_t)ll * r, 0.0), sig(r);
  for (int t = 0; t < r; ++t) sig[t] = std::sqrt(std::max(lam[t], 0.0));
  parallel_for(ls, [&](int64_t lo, int64_t hi) {
    for (int64_t i = lo; i < hi; ++i)
      for (int j = 0; j < K; ++j) {
        const double qv = Q[(size_t)i * K + j];
        for (int t = 0; t < r; ++t) Us[(size_t)i * r + t] += qv * V[(size_t)j * K + t];
      }
  }, 64);
  parallel_for(ll, [&](int64_t lo, int64_t hi) {
    for (int64_t i = lo; i < hi; ++i)
      for (int j = 0; j < K; ++j) {
        const double pv = P[(size_t)i * K + j];
        for (int t = 0; t < r; ++t) Ul[(size_t)i * r + t] += pv * V[(size_t)j * K + t];
      }
  }, 64);
  // L1 = U Sigma (m x r), L2 = V^T (r x n).  Wide (S = W~): U = Us, Sigma V^T =
  // Ul^T.  Tall (S = W~^T): V = Us, U Sigma = Ul.  Singular values that vanish
  // give zero columns / rows.  Sign: the largest-magnitude entry of each L1
  // column is positive.
  const double tiny = sig[0] * 1e-300;
  for (int t = 0; t < r; ++t) {
    const double s = sig[t];
    std::vector<double> u(m), v(n);
    if (S.wide()) {
      for (int i = 0; i < m; ++i) u[i] = Us[(size_t)i * r + t] * s;
      for (int j = 0; j < n; ++j) v[j] = s > tiny ? Ul[(size_t)j * r + t] / s : 0.0;
    } else {
      for (int i = 0; i < m; ++i) u[i] = Ul[(size_t)i * r + t];
      for (int j = 0; j < n; ++j) v[j] = Us[(size_t)j * r + t];
    }
    int imax = 0;
    for (int i = 1; i < m; ++i)
      if (std::fabs(u[i]) > std::fabs(u[imax])) imax = i;
    const double sgn = u[imax] < 0 ? -1.0 : 1.0;
    for (int i = 0; i < m; ++i) L1[(int64_t)i * r + t] = sgn * u[i];
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
