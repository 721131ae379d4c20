// Lloyd-Max codebook for one rotated coordinate, computed on the host.
//
// [NIK] "Step 1: random rotation", Lemma: a coordinate of a uniform point on
// S^{d-1} has density f_X(x) = C_d (1 - x^2)^((d-3)/2) on [-1, 1],
// C_d = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)).
// [NIK] "Step 2: optimal scalar quantization (Lloyd-Max)": alternate
// "boundaries = midpoints of neighbouring centroids" and "centroids =
// conditional means of their cells" until the centroids stop moving.
//
// Integration method: the substitution x = sin(theta) turns the cell integrals
// into int C_d cos^(d-2)(theta) {1, sin(theta)} dtheta, whose integrands are
// smooth for every d >= 3; each cell is split into sub-intervals sized to the
// density's width and integrated with 20-point Gauss-Legendre rules.
#include <cmath>
#include <cstdio>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "tq_internal.h"

namespace tq {
namespace {

struct GaussLegendre {
  static constexpr int n = 20;
  double x[n], w[n];
  GaussLegendre() {
    // Newton iteration on P_n for each root, standard initial guesses.
    for (int i = 0; i < n; ++i) {
      double z = std::cos(M_PI * (i + 0.75) / (n + 0.5));
      for (int it = 0; it < 100; ++it) {
        double p0 = 1.0, p1 = 0.0;
        for (int j = 1; j <= n; ++j) {
          double p2 = p1;
          p1 = p0;
          p0 = ((2.0 * j - 1.0) * z * p1 - (j - 1.0) * p2) / j;
        }
        double dp = n * (z * p0 - p1) / (z * z - 1.0);
        double dz = p0 / dp;
        z -= dz;
        if (std::fabs(dz) < 1e-17) break;
      }
      double p0 = 1.0, p1 = 0.0;
      for (int j = 1; j <= n; ++j) {
        double p2 = p1;
        p1 = p0;
        p0 = ((2.0 * j - 1.0) * z * p1 - (j - 1.0) * p2) / j;
      }
      double dp = n * (z * p0 - p1) / (z * z - 1.0);
      x[i] = z;
      w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
    }
  }
};

const GaussLegendre& gl() {
  static const GaussLegendre g;
  return g;
}

// Mass and first moment of f_X over [a, b] (both clipped to [-1, 1]).
void cell_moments(int d, double log_cd, double theta_max, double a, double b, double* m0,
                  double* m1) {
  a = std::fmax(-1.0, std::fmin(1.0, a));
  b = std::fmax(-1.0, std::fmin(1.0, b));
  double ta = std::asin(a), tb = std::asin(b);
  ta = std::fmax(ta, -theta_max);
  tb = std::fmin(tb, theta_max);
  *m0 = 0.0;
  *m1 = 0.0;
  if (!(tb > ta)) return;
  const double width = 1.0 / std::sqrt((double)d);
  int ns = (int)std::ceil((tb - ta) / width * 2.0);
  ns = ns < 1 ? 1 : (ns > 64 ? 64 : ns);
  const GaussLegendre& g = gl();
  const double h = (tb - ta) / ns;
  double s0 = 0.0, s1 = 0.0;
  for (int s = 0; s < ns; ++s) {
    const double lo = ta + s * h, mid = lo + 0.5 * h;
    for (int i = 0; i < GaussLegendre::n; ++i) {
      const double th = mid + 0.5 * h * g.x[i];
      const double c = std::cos(th);
      const double v = c > 0.0 ? std::exp(log_cd + (d - 2) * std::log(c)) : 0.0;
      s0 += g.w[i] * v;
      s1 += g.w[i] * v * std::sin(th);
    }
  }
  *m0 = 0.5 * h * s0;
  *m1 = 0.5 * h * s1;
}

float round_down_f32(double m) {
  float f = (float)m;
  if ((double)f > m) f = std::nextafter(f, -INFINITY);
  return f;
}

tq_status solve(int d, int planes, Codebook* cb) {
  cb->d = d;
  cb->planes = planes;
  const int K = 1 << planes;
  if (K == 1) {
    cb->centroids[0] = 0.0f;
    cb->cost = 1.0 / d;
    cb->n_walsh = 0;
    return TQ_OK;
  }
  const double log_cd = std::lgamma(d / 2.0) - std::lgamma((d - 1) / 2.0) - 0.5 * std::log(M_PI);
  // beyond theta_max the density is below 1e-300 relative to its scale
  double theta_max = M_PI / 2;
  if (d > 3) {
    double c = std::exp((-690.0 - log_cd) / (d - 2));
    if (c > 0.0 && c < 1.0) theta_max = std::acos(c);
  }
  // start from centroids spread evenly over +-2.5 standard deviations (1/sqrt(d)), inside (-1, 1)
  std::vector<double> c(K), cn(K), t(K + 1);
  const double spread = std::fmin(2.5 / std::sqrt((double)d), 1.0);
  for (int i = 0; i < K; ++i) c[i] = spread * ((2.0 * i + 1.0) / K - 1.0);
  int it = 0;
  for (it = 0; it < 2000000; ++it) {
    t[0] = -1.0;
    t[K] = 1.0;
    for (int i = 1; i < K; ++i) t[i] = 0.5 * (c[i - 1] + c[i]);
    double delta = 0.0;
    for (int i = 0; i < K; ++i) {
      double m0, m1;
      cell_moments(d, log_cd, theta_max, t[i], t[i + 1], &m0, &m1);
      if (!(m0 > 0.0)) return set_error(TQ_ERR_UNSUPPORTED, "codebook: empty Lloyd-Max cell");
      cn[i] = m1 / m0;
      delta = std::fmax(delta, std::fabs(cn[i] - c[i]));
    }
    c.swap(cn);
    if (delta < 1e-15) break;
  }
  // cost C(f_X, b) = sum over cells of int (x - c_i)^2 f = E[X^2] - sum c_i^2 P_i at the fixed point
  double cost = 1.0 / d;
  for (int i = 1; i < K; ++i) t[i] = 0.5 * (c[i - 1] + c[i]);
  for (int i = 0; i < K; ++i) {
    double m0, m1;
    cell_moments(d, log_cd, theta_max, t[i], t[i + 1], &m0, &m1);
    cost -= c[i] * c[i] * m0;
  }
  cb->cost = cost;
  // store as float32, exactly symmetric (the solution is symmetric up to rounding)
  for (int i = K / 2; i < K; ++i) {
    cb->centroids[i] = (float)c[i];
    cb->centroids[K - 1 - i] = -cb->centroids[i];
  }
  for (int i = 0; i + 1 < K; ++i) {
    const double mid = 0.5 * ((double)cb->centroids[i] + (double)cb->centroids[i + 1]);
    cb->thresholds[i] = round_down_f32(mid);
  }
  // odd Walsh expansion of the stored codebook
  cb->n_walsh = 0;
  for (int mask = 1; planes <= kMaxBits && mask < K; ++mask) {
    if (__builtin_popcount(mask) % 2 == 0) continue;
    double acc = 0.0;
    for (int idx = 0; idx < K; ++idx) {
      double sgn = 1.0;
      for (int p = 0; p < planes; ++p)
        if (mask >> p & 1) sgn *= ((idx >> p) & 1) ? 1.0 : -1.0;
      acc += sgn * (double)cb->centroids[idx];
    }
    cb->walsh_mask[cb->n_walsh] = mask;
    cb->walsh_coef[cb->n_walsh] = (float)(acc / K);
    cb->n_walsh++;
  }
  return TQ_OK;
}

}  // namespace

tq_status get_codebook(int d, int planes, const Codebook** out) {
  static std::mutex mu;
  static std::map<std::pair<int, int>, Codebook*> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto key = std::make_pair(d, planes);
  auto itr = cache.find(key);
  if (itr != cache.end()) {
    *out = itr->second;
    return TQ_OK;
  }
  Codebook* cb = new (std::nothrow) Codebook();
  if (!cb) return set_error(TQ_ERR_NO_MEMORY, "codebook: out of host memory");
  tq_status st = solve(d, planes, cb);
  if (st != TQ_OK) {
    delete cb;
    return st;
  }
  cache[key] = cb;
  *out = cb;
  return TQ_OK;
}

}  // namespace tq
