// Host-side tables of the quantizer: seeded Gaussian streams, the Haar
// rotation and the Lloyd-Max codebook of the Beta coordinate law.
//
// Page "TurboQuant 설명: 무엇인지와 LLM 메모리 6배 절약 구현 방법",
// section "1단계: 무작위 회전 + PolarQuant 압축": the rotation comes from the
// QR factorisation of a Gaussian matrix; after it, each coordinate of a unit
// vector follows Beta((d-1)/2, (d-1)/2) on [-1, 1], so the Lloyd-Max
// centroids for that law can be computed once per (dimension, bit width).
// Section "2단계: QJL 잔차 보정": the residual sketch uses a Gaussian
// projection S.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "tq.h"

namespace {

// ---------------------------------------------------------------- SplitMix64
// Steele, Lea and Flood (OOPSLA 2014): Weyl-sequence state, two xor-shift
// multiply rounds and a final xor-shift per output.
struct SplitMix64 {
  uint64_t s;
  uint64_t next() {
    s += 0x9E3779B97F4A7C15ull;
    uint64_t z = s;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  double uniform() { return ((double)(next() >> 11) + 0.5) * 0x1p-53; }
};

// Row-major rows x cols i.i.d. N(0,1) by Box-Muller (cos first).
void gaussian_fill(uint64_t seed, int kind, int64_t count, double *out) {
  SplitMix64 g{2 * seed + (uint64_t)kind};
  for (int64_t i = 0; i < count; i += 2) {
    double v1 = g.uniform();
    double v2 = g.uniform();
    double rad = std::sqrt(-2.0 * std::log(v1));
    double ang = 2.0 * M_PI * v2;
    out[i] = rad * std::cos(ang);
    if (i + 1 < count) out[i + 1] = rad * std::sin(ang);
  }
}

// Householder QR of the d x d row-major matrix a (overwritten); returns the
// orthogonal factor q (row-major) with every column flipped so that the
// matching diagonal entry of R is positive (sign(0) = +1).
void haar_from_gaussian(int d, std::vector<double> &a, std::vector<double> &q) {
  std::vector<double> vs((size_t)d * d, 0.0);  // Householder vectors, column k in vs[k*d..]
  std::vector<double> rdiag(d);
  for (int k = 0; k < d; ++k) {
    double norm2 = 0.0;
    for (int i = k; i < d; ++i) norm2 += a[(size_t)i * d + k] * a[(size_t)i * d + k];
    double norm = std::sqrt(norm2);
    double x0 = a[(size_t)k * d + k];
    double alpha = (x0 >= 0.0) ? -norm : norm;
    double *v = &vs[(size_t)k * d];
    for (int i = k; i < d; ++i) v[i] = a[(size_t)i * d + k];
    v[k] -= alpha;
    double vnorm2 = 0.0;
    for (int i = k; i < d; ++i) vnorm2 += v[i] * v[i];
    if (vnorm2 > 0.0) {
      double inv = 1.0 / std::sqrt(vnorm2);
      for (int i = k; i < d; ++i) v[i] *= inv;
      for (int j = k; j < d; ++j) {
        double dot = 0.0;
        for (int i = k; i < d; ++i) dot += v[i] * a[(size_t)i * d + j];
        for (int i = k; i < d; ++i) a[(size_t)i * d + j] -= 2.0 * v[i] * dot;
      }
    }
    rdiag[k] = a[(size_t)k * d + k];
  }
  // q = H_0 H_1 ... H_{d-1} applied to the identity.
  q.assign((size_t)d * d, 0.0);
  for (int i = 0; i < d; ++i) q[(size_t)i * d + i] = 1.0;
  for (int k = d - 1; k >= 0; --k) {
    const double *v = &vs[(size_t)k * d];
    for (int j = 0; j < d; ++j) {
      double dot = 0.0;
      for (int i = k; i < d; ++i) dot += v[i] * q[(size_t)i * d + j];
      if (dot == 0.0) continue;
      for (int i = k; i < d; ++i) q[(size_t)i * d + j] -= 2.0 * v[i] * dot;
    }
  }
  for (int j = 0; j < d; ++j) {
    if (rdiag[j] < 0.0)
      for (int i = 0; i < d; ++i) q[(size_t)i * d + j] = -q[(size_t)i * d + j];
  }
}

// ------------------------------------------------------ Beta-law quadrature
// Integrals over cells of f_d(x) = C (1 - x^2)^((d-3)/2) are taken in the
// angle x = sin(phi), where f_d(x) dx = C cos(phi)^(d-2) dphi is smooth for
// every d >= 3 (no endpoint singularity), with composite 20-point
// Gauss-Legendre on panels of width at most 0.25/sqrt(d) rad.
struct GaussLegendre {
  double x[20], w[20];
  GaussLegendre() {
    const int n = 20;
    for (int i = 0; i < n / 2; ++i) {
      double z = std::cos(M_PI * (i + 0.75) / (n + 0.5));
      double dp = 0.0;
      for (int it = 0; it < 100; ++it) {
        double p0 = 1.0, p1 = 0.0;
        for (int j = 1; j <= n; ++j) {
          double p2 = p1;
          p1 = p0;
          p0 = ((2.0 * j - 1.0) * z * p1 - (j - 1.0) * p2) / j;
        }
        dp = n * (z * p0 - p1) / (z * z - 1.0);
        double z1 = z;
        z = z1 - p0 / dp;
        if (std::fabs(z - z1) < 1e-16) break;
      }
      x[i] = -z;
      x[n - 1 - i] = z;
      w[i] = w[n - 1 - i] = 2.0 / ((1.0 - z * z) * dp * dp);
    }
  }
};

struct BetaLaw {
  int d;
  double log_c;   // log of the normalising constant (numerical)
  double panel;   // max panel width in phi
  double phi_max; // integration is cut beyond |phi| = phi_max (mass < 1e-300)
  GaussLegendre gl;

  explicit BetaLaw(int d_) : d(d_) {
    panel = 0.25 / std::sqrt((double)d);
    double xm = 40.0 / std::sqrt((double)d);
    phi_max = xm >= 1.0 ? 0.5 * M_PI : std::asin(xm);
    log_c = 0.0;
    double m0, m1, m2;
    raw(-1.0, 1.0, &m0, &m1, &m2);
    log_c = -std::log(m0);
  }
  double log_weight(double phi) const {  // log(cos(phi)^(d-2)) + log_c
    double c = std::cos(phi);
    if (c <= 0.0) return -INFINITY;
    return (d - 2) * std::log(c) + log_c;
  }
  // m0 = int f, m1 = int x f, m2 = int x^2 f over [a, b] (a, b in [-1, 1]).
  void raw(double a, double b, double *m0, double *m1, double *m2) const {
    double pa = std::asin(std::fmax(-1.0, std::fmin(1.0, a)));
    double pb = std::asin(std::fmax(-1.0, std::fmin(1.0, b)));
    pa = std::fmax(pa, -phi_max);
    pb = std::fmin(pb, phi_max);
    double s0 = 0.0, s1 = 0.0, s2 = 0.0;
    if (pb > pa) {
      int np = (int)std::ceil((pb - pa) / panel);
      if (np < 1) np = 1;
      double h = (pb - pa) / np;
      for (int p = 0; p < np; ++p) {
        double lo = pa + p * h;
        double mid = lo + 0.5 * h;
        for (int i = 0; i < 20; ++i) {
          double phi = mid + 0.5 * h * gl.x[i];
          double wgt = 0.5 * h * gl.w[i] * std::exp(log_weight(phi));
          double x = std::sin(phi);
          s0 += wgt;
          s1 += wgt * x;
          s2 += wgt * x * x;
        }
      }
    }
    *m0 = s0;
    *m1 = s1;
    *m2 = s2;
  }
  double pdf(double x) const {
    double v = 1.0 - x * x;
    if (v <= 0.0) return 0.0;
    // f(x) dx = C cos^(d-2) dphi and dx = cos(phi) dphi: f(x) = C cos^(d-3).
    return std::exp(0.5 * (d - 3) * std::log(v) + log_c);
  }
};

// One Lloyd update: c_k <- E[X | cell_k], cells split at the midpoints.
void lloyd_step(const BetaLaw &law, const std::vector<double> &c, std::vector<double> &out,
                std::vector<double> *mass) {
  int k = (int)c.size();
  out.resize(k);
  if (mass) mass->resize(k);
  for (int i = 0; i < k; ++i) {
    double lo = (i == 0) ? -1.0 : 0.5 * (c[i - 1] + c[i]);
    double hi = (i == k - 1) ? 1.0 : 0.5 * (c[i] + c[i + 1]);
    double m0, m1, m2;
    law.raw(lo, hi, &m0, &m1, &m2);
    out[i] = m1 / m0;
    if (mass) (*mass)[i] = m0;
  }
}

// Newton step on F(c) = c - T(c), T the Lloyd map.  dT/dc is tridiagonal:
// with cell [a, b] of centroid c_k and mass P,
//   dc_k/db = f(b) (b - c_k) / P,   dc_k/da = f(a) (c_k - a) / P,
// and a = (c_{k-1} + c_k)/2, b = (c_k + c_{k+1})/2.
bool newton_step(const BetaLaw &law, std::vector<double> &c) {
  int k = (int)c.size();
  std::vector<double> t, mass;
  lloyd_step(law, c, t, &mass);
  std::vector<double> lower(k, 0.0), diag(k, 1.0), upper(k, 0.0), rhs(k);
  for (int i = 0; i < k; ++i) {
    double lo = (i == 0) ? -1.0 : 0.5 * (c[i - 1] + c[i]);
    double hi = (i == k - 1) ? 1.0 : 0.5 * (c[i] + c[i + 1]);
    double d_hi = (i == k - 1) ? 0.0 : law.pdf(hi) * (hi - t[i]) / mass[i];
    double d_lo = (i == 0) ? 0.0 : law.pdf(lo) * (t[i] - lo) / mass[i];
    // Jacobian of F = I - dT/dc
    if (i > 0) lower[i] = -0.5 * d_lo;
    diag[i] = 1.0 - 0.5 * (d_lo + d_hi);
    if (i < k - 1) upper[i] = -0.5 * d_hi;
    rhs[i] = t[i] - c[i];  // -F
  }
  // Thomas algorithm.
  for (int i = 1; i < k; ++i) {
    if (diag[i - 1] == 0.0) return false;
    double m = lower[i] / diag[i - 1];
    diag[i] -= m * upper[i - 1];
    rhs[i] -= m * rhs[i - 1];
  }
  std::vector<double> delta(k);
  for (int i = k - 1; i >= 0; --i) {
    double v = rhs[i] - (i < k - 1 ? upper[i] * delta[i + 1] : 0.0);
    if (diag[i] == 0.0) return false;
    delta[i] = v / diag[i];
  }
  for (int i = 0; i < k; ++i) c[i] += delta[i];
  for (int i = 1; i < k; ++i)
    if (!(c[i] > c[i - 1])) return false;
  return c[0] > -1.0 && c[k - 1] < 1.0;
}

}  // namespace

extern "C" tq_status tq_make_rotation(int32_t d, uint64_t seed, int32_t kind, double *out) {
  if (out == nullptr || d < 2 || d > 4096) return TQ_ERR_INVALID;
  if (kind != TQ_KIND_PI && kind != TQ_KIND_S && kind != TQ_KIND_M) return TQ_ERR_INVALID;
  size_t n = (size_t)d * d;
  if (kind == TQ_KIND_S) {
    gaussian_fill(seed, 1, (int64_t)n, out);
    return TQ_OK;
  }
  std::vector<double> g(n), pi;
  gaussian_fill(seed, 0, (int64_t)n, g.data());
  haar_from_gaussian(d, g, pi);
  if (kind == TQ_KIND_PI) {
    std::memcpy(out, pi.data(), n * sizeof(double));
    return TQ_OK;
  }
  std::vector<double> s(n);
  gaussian_fill(seed, 1, (int64_t)n, s.data());
  for (int i = 0; i < d; ++i)       // M[i][j] = sum_k S[i][k] Pi[j][k]
    for (int j = 0; j < d; ++j) {
      double acc = 0.0;
      for (int k = 0; k < d; ++k) acc += s[(size_t)i * d + k] * pi[(size_t)j * d + k];
      out[(size_t)i * d + j] = acc;
    }
  return TQ_OK;
}

extern "C" tq_status tq_make_codebook(int32_t d, int32_t bits, double *centroids,
                                      double *boundaries, double *mse_per_coord) {
  if (centroids == nullptr || boundaries == nullptr) return TQ_ERR_INVALID;
  if (d < 3 || d > (1 << 20) || bits < 1 || bits > 8) return TQ_ERR_INVALID;
  const int k = 1 << bits;
  BetaLaw law(d);
  // Start at the (i + 1/2)/K quantiles of the standard normal scaled by
  // 1/sqrt(d) (clamped into (-1, 1)); Lloyd steps then Newton steps.
  std::vector<double> c(k), t;
  for (int i = 0; i < k; ++i) {
    double p = (i + 0.5) / k;
    // inverse normal CDF by bisection on erfc (init only)
    double lo = -10.0, hi = 10.0;
    for (int it = 0; it < 200; ++it) {
      double mid = 0.5 * (lo + hi);
      if (0.5 * std::erfc(-mid / std::sqrt(2.0)) < p) lo = mid; else hi = mid;
    }
    double v = 0.5 * (lo + hi) / std::sqrt((double)d);
    c[i] = std::fmax(-0.999, std::fmin(0.999, v));
  }
  for (int it = 0; it < 200; ++it) {
    lloyd_step(law, c, t, nullptr);
    c.swap(t);
  }
  bool converged = false;
  for (int it = 0; it < 100 && !converged; ++it) {
    std::vector<double> prev = c;
    if (!newton_step(law, c)) return TQ_ERR_NO_CONVERGENCE;
    double step = 0.0;
    for (int i = 0; i < k; ++i) step = std::fmax(step, std::fabs(c[i] - prev[i]));
    if (step < 1e-15) converged = true;
  }
  if (!converged) return TQ_ERR_NO_CONVERGENCE;
  // The law is symmetric and log-concave, so the fixed point is unique and
  // symmetric; remove rounding noise so the middle boundary is exactly 0.
  for (int i = 0; i < k / 2; ++i) {
    double m = 0.5 * (c[k - 1 - i] - c[i]);
    c[k - 1 - i] = m;
    c[i] = -m;
  }
  for (int i = 0; i < k; ++i) centroids[i] = c[i];
  for (int i = 0; i + 1 < k; ++i) boundaries[i] = 0.5 * (c[i] + c[i + 1]);
  if (mse_per_coord) {
    double mse = 0.0;
    for (int i = 0; i < k; ++i) {
      double lo = (i == 0) ? -1.0 : boundaries[i - 1];
      double hi = (i == k - 1) ? 1.0 : boundaries[i];
      double m0, m1, m2;
      law.raw(lo, hi, &m0, &m1, &m2);
      mse += m2 - 2.0 * c[i] * m1 + c[i] * c[i] * m0;
    }
    *mse_per_coord = mse;
  }
  return TQ_OK;
}

// ------------------------------------------------------- polar angle laws
// PolarQuant variant (page section "1단계", the recursive polar transform):
// at level l >= 2 an angle splits two radii that span k = 2^(l-1)
// dimensions each; for a uniform point on the sphere its density on
// [0, pi/2] is proportional to (sin t cos t)^(k-1).  Moments over a cell
// by composite 20-point Gauss-Legendre in t (panels of width at most
// 0.05/sqrt(k)), normalised numerically; 2-bit Lloyd-Max codebooks by Lloyd
// iteration from the quantiles of a fine table, made exactly symmetric
// about pi/4 at the end.
namespace {

struct AngleLaw {
  int k;
  double log_c = 0.0;
  double panel;
  GaussLegendre gl;
  explicit AngleLaw(int k_) : k(k_) {
    panel = 0.05 / std::sqrt((double)k);
    double m0, m1;
    raw(0.0, 0.5 * M_PI, &m0, &m1);
    log_c = -std::log(m0);
  }
  void raw(double a, double b, double *m0, double *m1) const {
    double s0 = 0.0, s1 = 0.0;
    if (b > a) {
      int np = (int)std::ceil((b - a) / panel);
      if (np < 1) np = 1;
      const double h = (b - a) / np;
      for (int p = 0; p < np; ++p) {
        const double mid = a + (p + 0.5) * h;
        for (int i = 0; i < 20; ++i) {
          const double t = mid + 0.5 * h * gl.x[i];
          const double sc = std::sin(t) * std::cos(t);
          const double f = sc > 0.0 ? std::exp((k - 1) * std::log(sc) + log_c) : (k == 1 ? std::exp(log_c) : 0.0);
          const double wgt = 0.5 * h * gl.w[i] * f;
          s0 += wgt;
          s1 += wgt * t;
        }
      }
    }
    *m0 = s0;
    *m1 = s1;
  }
};

}  // namespace

extern "C" tq_status tq_make_polar_codebook(int32_t d, double *centroids, double *boundaries) {
  if (centroids == nullptr || boundaries == nullptr) return TQ_ERR_INVALID;
  int levels = 0;
  while ((1 << levels) < d) ++levels;
  if (d < 64 || (1 << levels) != d || levels > 20) return TQ_ERR_INVALID;
  for (int lv = 2; lv <= levels; ++lv) {
    const AngleLaw law(1 << (lv - 1));
    // start from the quantiles (i + 1/2)/4 of a 4096-point cdf table
    double c[4];
    {
      const int n = 4096;
      double acc = 0.0;
      int q = 0;
      for (int i = 0; i < n && q < 4; ++i) {
        const double a = 0.5 * M_PI * i / n, b = 0.5 * M_PI * (i + 1) / n;
        double m0, m1;
        law.raw(a, b, &m0, &m1);
        acc += m0;
        while (q < 4 && acc >= (q + 0.5) / 4.0) c[q++] = b;
      }
      while (q < 4) c[q++] = 0.5 * M_PI;
    }
    bool done = false;
    for (int it = 0; it < 100000 && !done; ++it) {
      double nc[4], step = 0.0;
      for (int i = 0; i < 4; ++i) {
        const double lo = i == 0 ? 0.0 : 0.5 * (c[i - 1] + c[i]);
        const double hi = i == 3 ? 0.5 * M_PI : 0.5 * (c[i] + c[i + 1]);
        double m0, m1;
        law.raw(lo, hi, &m0, &m1);
        if (!(m0 > 0.0)) return TQ_ERR_NO_CONVERGENCE;
        nc[i] = m1 / m0;
        step = std::fmax(step, std::fabs(nc[i] - c[i]));
      }
      for (int i = 0; i < 4; ++i) c[i] = nc[i];
      done = step < 1e-15;
    }
    if (!done) return TQ_ERR_NO_CONVERGENCE;
    for (int i = 0; i < 2; ++i) {
      const double m = 0.5 * (c[i] + (0.5 * M_PI - c[3 - i]));
      c[i] = m;
      c[3 - i] = 0.5 * M_PI - m;
    }
    for (int i = 0; i < 4; ++i) centroids[4 * (lv - 2) + i] = c[i];
    for (int i = 0; i < 3; ++i) boundaries[3 * (lv - 2) + i] = 0.5 * (c[i] + c[i + 1]);
  }
  return TQ_OK;
}

extern "C" const char *tq_status_string(tq_status s) {
  switch (s) {
    case TQ_OK: return "ok";
    case TQ_ERR_INVALID: return "invalid argument";
    case TQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case TQ_ERR_NO_CONVERGENCE: return "Lloyd-Max solver did not converge";
    case TQ_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}
