// Host-side set-up of the rotation and the codebooks: pure C++, no device work.
//
// tq_build_codebook: Lloyd-Max quantizer for one rotated coordinate, fitted once per
//   (D, bits, family) and shared (turboquant-serve 0.1.2, "Architecture": the codebook is
//   MSE-optimal for the Beta prior on rotated unit vectors and fitted once; TorbuQuant docs,
//   "Current Status": exact Beta-sphere and Gaussian-approximation codebooks).
// tq_rht_signs: the sign vector of the randomized Hadamard rotation (tq-kv, "Quick Start":
//   generate_signs(dim, seed)), drawn with SplitMix64.
//
// The solver alternates the midpoint condition t_j = (c_{j-1} + c_j)/2 and the centroid
// condition c_j = E[X | t_j < X <= t_{j+1}] (Lloyd), then polishes the same fixed point with
// Newton steps on the boundary equations (tridiagonal Jacobian), keeping the codebook exactly
// symmetric.  Cell probabilities use the regularized incomplete beta function (own continued
// fraction, Lentz's method) or erfc; partial first moments are closed form.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "../../include/tq.h"
#include "tq_internal.h"

namespace {

// ---------------------------------------------------------------------------------------------
// Regularized incomplete beta I_x(a, b) by its continued fraction (Abramowitz & Stegun 26.5.8),
// evaluated with the modified Lentz method.  Only used with x <= (a+1)/(a+b+2), where the
// fraction converges quickly; callers use the symmetry I_x(a,b) = 1 - I_{1-x}(b,a) otherwise.
// ---------------------------------------------------------------------------------------------
double beta_cf(double a, double b, double x) {
  const double tiny = 1e-300;
  const double eps = 1e-17;
  double c = 1.0;
  double d = 1.0 - (a + b) * x / (a + 1.0);
  if (std::fabs(d) < tiny) d = tiny;
  d = 1.0 / d;
  double f = d;
  for (int m = 1; m < 100000; ++m) {
    // even term d_{2m}
    double num = m * (b - m) * x / ((a + 2.0 * m - 1.0) * (a + 2.0 * m));
    d = 1.0 + num * d;
    if (std::fabs(d) < tiny) d = tiny;
    c = 1.0 + num / c;
    if (std::fabs(c) < tiny) c = tiny;
    d = 1.0 / d;
    f *= d * c;
    // odd term d_{2m+1}
    num = -(a + m) * (a + b + m) * x / ((a + 2.0 * m) * (a + 2.0 * m + 1.0));
    d = 1.0 + num * d;
    if (std::fabs(d) < tiny) d = tiny;
    c = 1.0 + num / c;
    if (std::fabs(c) < tiny) c = tiny;
    d = 1.0 / d;
    const double delta = d * c;
    f *= delta;
    if (std::fabs(delta - 1.0) < eps) break;
  }
  return f;
}

double reg_inc_beta(double a, double b, double x) {
  if (x <= 0.0) return 0.0;
  if (x >= 1.0) return 1.0;
  const double log_front = a * std::log(x) + b * std::log1p(-x) - std::log(a) -
                           (std::lgamma(a) + std::lgamma(b) - std::lgamma(a + b));
  if (x < (a + 1.0) / (a + b + 2.0)) return std::exp(log_front) * beta_cf(a, b, x);
  const double log_front_c = b * std::log1p(-x) + a * std::log(x) - std::log(b) -
                             (std::lgamma(a) + std::lgamma(b) - std::lgamma(a + b));
  return 1.0 - std::exp(log_front_c) * beta_cf(b, a, 1.0 - x);
}

// One coordinate law: cdf F, survival S, pdf f, integral of x f over [lo, hi], E[X^2].
struct Law {
  int family;
  double D;
  double a;        // Beta shape (D-1)/2
  double expo;     // (D-3)/2
  double logC;     // log normaliser of the sphere density
  double sigma;    // Gaussian sigma
  double lo, hi;   // support

  explicit Law(int fam, int dim) : family(fam), D(dim) {
    a = (D - 1.0) / 2.0;
    expo = (D - 3.0) / 2.0;
    logC = std::lgamma(D / 2.0) - 0.5 * std::log(M_PI) - std::lgamma((D - 1.0) / 2.0);
    sigma = 1.0 / std::sqrt(D);
    if (family == TQ_CODEBOOK_BETA) {
      lo = -1.0;
      hi = 1.0;
    } else {
      lo = -INFINITY;
      hi = INFINITY;
    }
  }
  double cdf(double x) const {
    if (family == TQ_CODEBOOK_BETA) {
      if (x <= -1.0) return 0.0;
      if (x >= 1.0) return 1.0;
      return reg_inc_beta(a, a, 0.5 * (1.0 + x));
    }
    return 0.5 * std::erfc(-x / (sigma * M_SQRT2));
  }
  double sf(double x) const {
    if (family == TQ_CODEBOOK_BETA) {
      if (x <= -1.0) return 1.0;
      if (x >= 1.0) return 0.0;
      return reg_inc_beta(a, a, 0.5 * (1.0 - x));
    }
    return 0.5 * std::erfc(x / (sigma * M_SQRT2));
  }
  double pdf(double x) const {
    if (family == TQ_CODEBOOK_BETA) {
      const double w = 1.0 - x * x;
      return w <= 0.0 ? 0.0 : std::exp(logC + expo * std::log(w));
    }
    const double z = x / sigma;
    return std::exp(-0.5 * z * z) / (sigma * std::sqrt(2.0 * M_PI));
  }
  // integral of x f(x) over [l, h]
  double first_moment(double l, double h) const {
    if (family == TQ_CODEBOOK_BETA) {
      const double k = expo + 1.0;
      auto g = [&](double x) {
        const double w = 1.0 - x * x;
        return w <= 0.0 ? 0.0 : std::exp(k * std::log(w));
      };
      return std::exp(logC) * (g(l) - g(h)) / (2.0 * k);
    }
    auto f = [&](double x) { return std::isfinite(x) ? pdf(x) : 0.0; };
    return sigma * sigma * (f(l) - f(h));
  }
  double second_moment() const { return family == TQ_CODEBOOK_BETA ? 1.0 / D : sigma * sigma; }
  // quantile by bisection on the cdf (only used for start points)
  double ppf(double p) const {
    double l = family == TQ_CODEBOOK_BETA ? -1.0 : -40.0 * sigma;
    double h = -l;
    for (int i = 0; i < 200; ++i) {
      const double m = 0.5 * (l + h);
      if (cdf(m) < p) l = m; else h = m;
    }
    return 0.5 * (l + h);
  }
};

// centroids and cell probabilities for inner boundaries t[0..L-2]
void centroids_for(const Law& law, const std::vector<double>& t, std::vector<double>& c,
                   std::vector<double>& P) {
  const int L = (int)t.size() + 1;
  c.resize(L);
  P.resize(L);
  for (int j = 0; j < L; ++j) {
    const double l = j == 0 ? law.lo : t[j - 1];
    const double h = j == L - 1 ? law.hi : t[j];
    double p;
    if (h <= 0.0) p = law.cdf(h) - law.cdf(l);
    else p = law.sf(l) - law.sf(h);
    P[j] = p;
    c[j] = law.first_moment(l, h) / p;
  }
}

void symmetrize(std::vector<double>& c) {
  const int L = (int)c.size();
  std::vector<double> s(L);
  for (int j = 0; j < L; ++j) s[j] = 0.5 * (c[j] - c[L - 1 - j]);
  c = s;
}

std::vector<double> mids(const std::vector<double>& c) {
  std::vector<double> t(c.size() - 1);
  for (size_t j = 0; j + 1 < c.size(); ++j) t[j] = 0.5 * (c[j] + c[j + 1]);
  return t;
}

double max_abs_diff(const std::vector<double>& a, const std::vector<double>& b) {
  double m = 0.0;
  for (size_t i = 0; i < a.size(); ++i) m = std::fmax(m, std::fabs(a[i] - b[i]));
  return m;
}

// Newton step on G_j(t) = t_j - (c_{j-1}(t) + c_j(t))/2, solved with the Thomas algorithm.
std::vector<double> newton_step(const Law& law, const std::vector<double>& t) {
  const int n = (int)t.size();
  std::vector<double> c, P;
  centroids_for(law, t, c, P);
  std::vector<double> lower(n), diag(n), upper(n), rhs(n);
  for (int k = 0; k < n; ++k) {
    const double f = law.pdf(t[k]);
    const double dcu = f * (t[k] - c[k]) / P[k];          // d c_k     / d t_k (upper end)
    const double dcl = f * (c[k + 1] - t[k]) / P[k + 1];  // d c_{k+1} / d t_k (lower end)
    rhs[k] = t[k] - 0.5 * (c[k] + c[k + 1]);
    diag[k] = 1.0 - 0.5 * (dcu + dcl);
    // row k+1 depends on t_k through c_{k+1}; row k-1 on t_k through c_k
    if (k + 1 < n) lower[k + 1] = -0.5 * dcl;
    if (k - 1 >= 0) upper[k - 1] = -0.5 * dcu;
  }
  // Thomas: solve lower[k] x[k-1] + diag[k] x[k] + upper[k] x[k+1] = rhs[k]
  for (int k = 1; k < n; ++k) {
    const double w = lower[k] / diag[k - 1];
    diag[k] -= w * upper[k - 1];
    rhs[k] -= w * rhs[k - 1];
  }
  std::vector<double> x(n);
  x[n - 1] = rhs[n - 1] / diag[n - 1];
  for (int k = n - 2; k >= 0; --k) x[k] = (rhs[k] - upper[k] * x[k + 1]) / diag[k];
  return x;
}

uint64_t splitmix64_next(uint64_t& state) {
  state += 0x9E3779B97F4A7C15ull;
  uint64_t z = state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

}  // namespace

// Sign bits of the rotation: bit i of the returned words set means s_i = -1.
void tq_sign_words(int32_t D, uint64_t seed, uint64_t* words, int nwords) {
  for (int w = 0; w < nwords; ++w) words[w] = 0;
  uint64_t state = seed;
  for (int i = 0; i < D; ++i) {
    const uint64_t z = splitmix64_next(state);
    if (z >> 63) words[i >> 6] |= 1ull << (i & 63);
  }
}

extern "C" int tq_rht_signs(int32_t D, uint64_t seed, int8_t* out) {
  if (out == nullptr || D < 1 || D > 65536) return TQ_ERR_INVALID_ARG;
  uint64_t state = seed;
  for (int i = 0; i < D; ++i) out[i] = (splitmix64_next(state) >> 63) ? -1 : 1;
  return TQ_OK;
}

extern "C" int tq_build_codebook(int32_t D, int32_t bits, int32_t family, float* centroids,
                                 float* boundaries, double* centroids_f64, double* boundaries_f64,
                                 double* mse) {
  if (centroids == nullptr || boundaries == nullptr) return TQ_ERR_INVALID_ARG;
  if (D < 2 || D > 65536 || bits < 1 || bits > 8) return TQ_ERR_INVALID_ARG;
  if (family != TQ_CODEBOOK_BETA && family != TQ_CODEBOOK_GAUSSIAN) return TQ_ERR_INVALID_ARG;
  if (family == TQ_CODEBOOK_BETA && D < 3) return TQ_ERR_UNSUPPORTED;
  const double tol = 1e-13;
  const Law law(family, D);
  const int L = 1 << bits;

  std::vector<double> c(L), t, P, cn;
  for (int j = 0; j < L; ++j) c[j] = law.ppf((j + 0.5) / L);
  symmetrize(c);
  double residual = INFINITY;
  for (int it = 0; it < 400 && residual > tol; ++it) {
    t = mids(c);
    centroids_for(law, t, cn, P);
    symmetrize(cn);
    residual = max_abs_diff(cn, c);
    c = cn;
  }
  // Newton runs to the floating-point floor, not just to `tol`, so the fp32 rounding of the fixed
  // point does not depend on where an iteration happened to stop.
  if (residual > tol || bits >= 3) {
    t = mids(c);
    double best = residual;
    int stall = 0;
    for (int it = 0; it < 60 && residual > 1e-17 && stall < 3; ++it) {
      const std::vector<double> step = newton_step(law, t);
      double lam = 1.0;
      std::vector<double> tt(t.size());
      for (int tries = 0; tries < 60; ++tries) {
        for (size_t k = 0; k < t.size(); ++k) tt[k] = t[k] - lam * step[k];
        std::vector<double> s(tt.size());
        for (size_t k = 0; k < tt.size(); ++k) s[k] = 0.5 * (tt[k] - tt[tt.size() - 1 - k]);
        tt = s;
        bool ordered = tt.front() > law.lo && tt.back() < law.hi;
        for (size_t k = 0; k + 1 < tt.size(); ++k) ordered = ordered && tt[k] < tt[k + 1];
        if (ordered) break;
        lam *= 0.5;
      }
      t = tt;
      centroids_for(law, t, cn, P);
      symmetrize(cn);
      std::vector<double> chk;
      centroids_for(law, mids(cn), chk, P);
      symmetrize(chk);
      residual = max_abs_diff(chk, cn);
      c = cn;
      if (residual < best) {
        best = residual;
        stall = 0;
      } else {
        ++stall;
      }
    }
  }
  t = mids(c);
  t[L / 2 - 1] = 0.0;
  centroids_for(law, t, cn, P);
  residual = max_abs_diff(cn, c);
  if (!(residual <= 1e-12)) return TQ_ERR_NO_CONVERGENCE;

  double m = law.second_moment();
  for (int j = 0; j < L; ++j) m -= P[j] * c[j] * c[j];
  for (int j = 0; j < L; ++j) centroids[j] = (float)c[j];
  for (int j = 0; j + 1 < L; ++j) boundaries[j] = (float)t[j];
  if (centroids_f64) std::memcpy(centroids_f64, c.data(), sizeof(double) * L);
  if (boundaries_f64) std::memcpy(boundaries_f64, t.data(), sizeof(double) * (L - 1));
  if (mse) *mse = m;
  return TQ_OK;
}
