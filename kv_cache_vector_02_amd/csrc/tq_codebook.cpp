// Lloyd-Max codebook for one coordinate of a uniformly rotated unit vector.
//
// Density (blog notes on the TurboQuant paper, Lemma 1):
//   f(x) = C_d (1 - x^2)^((d-3)/2) on [-1, 1],  C_d = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)).
// Optimal scalar quantizer = 1-D continuous k-means (eq. (4) of the same
// notes), found by the Lloyd-Max iteration (explainer page, section 5):
// boundaries at midpoints of adjacent centroids, centroids at the
// conditional means of their cells.
//
// Integration is done in theta = asin(x), where f(x) dx = C_d cos^(d-2)(theta)
// dtheta is smooth for every d >= 2 (no endpoint singularity), with composite
// 16-point Gauss-Legendre panels of width ~ sigma/8 and a cumulative table, so
// each Lloyd step costs O(2^b) panel evaluations.  d == 0 is the N(0,1) limit
// with erfc and the Gaussian density in closed form.
#include <cmath>
#include <vector>

#include "tq_internal.h"

namespace tq {
namespace {

// 16-point Gauss-Legendre nodes/weights on [-1, 1] (symmetric halves).
const double kGLx[8] = {0.0950125098376374401853193, 0.2816035507792589132304605,
                        0.4580167776572273863424194, 0.6178762444026437484466718,
                        0.7554044083550030338951012, 0.8656312023878317438804679,
                        0.9445750230732325760779884, 0.9894009349916499325961542};
const double kGLw[8] = {0.1894506104550684962853967, 0.1826034150449235888667637,
                        0.1691565193950025381893121, 0.1495959888165767320815017,
                        0.1246289712555338720524763, 0.0951585116824927848099251,
                        0.0622535239386478928628438, 0.0271524594117540948517806};

struct Half {  // integrals over the upper half line
  virtual double mass(double a, double b) const = 0;      // P(a <= X < b), 0 <= a <= b
  virtual double moment(double a, double b) const = 0;    // int_a^b x f(x) dx
  virtual ~Half() {}
};

struct GaussHalf : Half {
  double mass(double a, double b) const override {
    const double s = 1.0 / std::sqrt(2.0);
    double eb = std::isinf(b) ? 0.0 : std::erfc(b * s);
    return 0.5 * (std::erfc(a * s) - eb);
  }
  double moment(double a, double b) const override {
    const double k = 1.0 / std::sqrt(2.0 * M_PI);
    double pb = std::isinf(b) ? 0.0 : std::exp(-0.5 * b * b);
    return k * (std::exp(-0.5 * a * a) - pb);
  }
};

struct SphereHalf : Half {
  int d;
  double logc, h, tmax;
  std::vector<double> cum_m, cum_x;  // cumulative integrals at theta = k h

  explicit SphereHalf(int d_) : d(d_) {
    logc = std::lgamma(0.5 * d) - 0.5 * std::log(M_PI) - std::lgamma(0.5 * (d - 1));
    const double sigma = 1.0 / std::sqrt((double)d);
    h = std::fmin(sigma, 0.25) / 8.0;
    // past tmax the integrand is below 1e-300 of its peak
    double t = M_PI / 2;
    if (d > 2) {
      double c = std::exp(-700.0 / (double)(d - 2));
      t = std::fmin(M_PI / 2, std::acos(c));
    }
    tmax = t;
    int K = (int)std::ceil(tmax / h);
    h = tmax / K;
    cum_m.assign(K + 1, 0.0);
    cum_x.assign(K + 1, 0.0);
    for (int k = 0; k < K; ++k) {
      double m, x;
      panel(k * h, (k + 1) * h, &m, &x);
      cum_m[k + 1] = cum_m[k] + m;
      cum_x[k + 1] = cum_x[k] + x;
    }
  }
  // density in theta: C cos^(d-2) t ; first moment integrand: sin t * that
  double w(double t) const {
    double c = std::cos(t);
    if (c <= 0) return 0.0;
    return std::exp(logc + (d - 2) * std::log(c));
  }
  void panel(double a, double b, double* m, double* x) const {
    double mid = 0.5 * (a + b), half = 0.5 * (b - a);
    double sm = 0, sx = 0;
    for (int i = 0; i < 8; ++i) {
      for (int sgn = -1; sgn <= 1; sgn += 2) {
        double t = mid + sgn * half * kGLx[i];
        double v = w(t);
        sm += kGLw[i] * v;
        sx += kGLw[i] * v * std::sin(t);
      }
    }
    *m = sm * half;
    *x = sx * half;
  }
  // cumulative integrals from theta = 0 to theta
  void cum(double t, double* m, double* x) const {
    if (t >= tmax) {
      *m = cum_m.back();
      *x = cum_x.back();
      return;
    }
    int k = (int)std::floor(t / h);
    if (k >= (int)cum_m.size() - 1) k = (int)cum_m.size() - 2;
    double pm = 0, px = 0;
    if (t > k * h) panel(k * h, t, &pm, &px);
    *m = cum_m[k] + pm;
    *x = cum_x[k] + px;
  }
  double mass(double a, double b) const override {
    double ma, xa, mb, xb;
    cum(std::asin(std::fmin(a, 1.0)), &ma, &xa);
    cum(std::asin(std::fmin(b, 1.0)), &mb, &xb);
    return mb - ma;
  }
  double moment(double a, double b) const override {
    double ma, xa, mb, xb;
    cum(std::asin(std::fmin(a, 1.0)), &ma, &xa);
    cum(std::asin(std::fmin(b, 1.0)), &mb, &xb);
    return xb - xa;
  }
};

// Lloyd-Max on the upper half line of an even density: H centroids in
// (0, top), the first cell starting at 0 (the middle boundary of the full
// codebook), iterated until the largest move is below tol * sigma or
// rounding noise dominates.
std::vector<double> lloyd_half(const Half& f, int H, double sigma, double top) {
  std::vector<double> c(H), cn(H), e(H + 1);
  for (int i = 0; i < H; ++i) c[i] = std::fmin(sigma * 3.0 * (i + 0.5) / H, 0.999 * top);
  const double tol = 1e-13;
  double best_move = INFINITY;
  int since_best = 0;
  for (int it = 0; it < 1000000; ++it) {
    e[0] = 0.0;
    for (int i = 1; i < H; ++i) e[i] = 0.5 * (c[i - 1] + c[i]);
    e[H] = top;
    double move = 0;
    for (int i = 0; i < H; ++i) {
      double m = f.mass(e[i], e[i + 1]);
      cn[i] = m > 0 ? f.moment(e[i], e[i + 1]) / m : c[i];
      move = std::fmax(move, std::fabs(cn[i] - c[i]) / sigma);
    }
    c.swap(cn);
    if (move < tol) break;
    // stop once rounding noise dominates: no new minimum for a long stretch
    if (move < best_move) {
      best_move = move;
      since_best = 0;
    } else if (++since_best > 2000 && best_move < 1e-10) {
      break;
    }
  }
  return c;
}

// The law of a level-l angle psi of the recursive polar transform, in
// t = 2 psi - pi/2 on [-pi/2, pi/2]: with a = 2^(l-2), sin^2 psi ~ Beta(a, a)
// gives the density of psi proportional to sin^(2a-1)(2 psi), i.e. cos^k(t)
// with k = 2a - 1 (even in t).  Integrals over the upper half in t, unnormalised
// (only the cells' conditional means are needed), on cumulative 16-point
// Gauss-Legendre panels.
struct AngleHalf : Half {
  double k, h, tmax;
  std::vector<double> cum_m, cum_x;

  explicit AngleHalf(double k_) : k(k_) {
    const double sigma = 1.0 / std::sqrt(k + 1.0);
    h = std::fmin(sigma, 0.25) / 8.0;
    tmax = k > 0 ? std::fmin(M_PI / 2, std::acos(std::exp(-700.0 / k))) : M_PI / 2;
    int K = (int)std::ceil(tmax / h);
    h = tmax / K;
    cum_m.assign(K + 1, 0.0);
    cum_x.assign(K + 1, 0.0);
    for (int i = 0; i < K; ++i) {
      double m, x;
      panel(i * h, (i + 1) * h, &m, &x);
      cum_m[i + 1] = cum_m[i] + m;
      cum_x[i + 1] = cum_x[i] + x;
    }
  }
  double w(double t) const {
    double c = std::cos(t);
    return c <= 0 ? 0.0 : std::exp(k * std::log(c));
  }
  void panel(double a, double b, double* m, double* x) const {
    double mid = 0.5 * (a + b), half = 0.5 * (b - a);
    double sm = 0, sx = 0;
    for (int i = 0; i < 8; ++i) {
      for (int sgn = -1; sgn <= 1; sgn += 2) {
        double t = mid + sgn * half * kGLx[i];
        double v = w(t);
        sm += kGLw[i] * v;
        sx += kGLw[i] * v * t;
      }
    }
    *m = sm * half;
    *x = sx * half;
  }
  void cum(double t, double* m, double* x) const {
    if (t >= tmax) {
      *m = cum_m.back();
      *x = cum_x.back();
      return;
    }
    int i = (int)std::floor(t / h);
    if (i >= (int)cum_m.size() - 1) i = (int)cum_m.size() - 2;
    double pm = 0, px = 0;
    if (t > i * h) panel(i * h, t, &pm, &px);
    *m = cum_m[i] + pm;
    *x = cum_x[i] + px;
  }
  double mass(double a, double b) const override {
    double ma, xa, mb, xb;
    cum(a, &ma, &xa);
    cum(b, &mb, &xb);
    return mb - ma;
  }
  double moment(double a, double b) const override {
    double ma, xa, mb, xb;
    cum(a, &ma, &xa);
    cum(b, &mb, &xb);
    return xb - xa;
  }
};

}  // namespace

tq_status build_codebook(int d, int bits, double* centroids, double* boundaries) {
  const int K = 1 << bits;
  const int H = K / 2;
  const double sigma = d == 0 ? 1.0 : 1.0 / std::sqrt((double)d);
  const double top = d == 0 ? INFINITY : 1.0;
  GaussHalf gh;
  SphereHalf* sh = d == 0 ? nullptr : new SphereHalf(d);
  const Half& f = d == 0 ? (const Half&)gh : (const Half&)*sh;
  std::vector<double> c = lloyd_half(f, H, sigma, top);
  delete sh;
  for (int i = 0; i < H; ++i) {
    centroids[H + i] = c[i];
    centroids[H - 1 - i] = -c[i];
  }
  boundaries[H - 1] = 0.0;
  for (int i = 1; i < H; ++i) {
    double b = 0.5 * (c[i - 1] + c[i]);
    boundaries[H - 1 + i] = b;
    boundaries[H - 1 - i] = -b;
  }
  return TQ_OK;
}

// Level 1: the angle is uniform on (-pi, pi], whose Lloyd-Max quantizer is
// the uniform grid (cells of width 2 pi / K from -pi, centroids at their
// middles).  Levels >= 2: the law above, solved in t and mapped back with
// psi = (t + pi/2) / 2; the codebook is symmetric about pi/4.
tq_status build_polar_codebook(int level, int bits, double* centroids, double* boundaries) {
  const int K = 1 << bits;
  if (level == 1) {
    const double w = 2 * M_PI / K;
    for (int i = 0; i < K; ++i) centroids[i] = -M_PI + (i + 0.5) * w;
    for (int i = 1; i < K; ++i) boundaries[i - 1] = -M_PI + i * w;
    return TQ_OK;
  }
  const int H = K / 2;
  const double k = std::ldexp(1.0, level - 1) - 1.0;
  AngleHalf f(k);
  std::vector<double> c = lloyd_half(f, H, 1.0 / std::sqrt(k + 1.0), M_PI / 2);
  auto psi = [](double t) { return 0.5 * (t + M_PI / 2); };
  for (int i = 0; i < H; ++i) {
    centroids[H + i] = psi(c[i]);
    centroids[H - 1 - i] = psi(-c[i]);
  }
  boundaries[H - 1] = M_PI / 4;
  for (int i = 1; i < H; ++i) {
    double b = 0.5 * (c[i - 1] + c[i]);
    boundaries[H - 1 + i] = psi(b);
    boundaries[H - 1 - i] = psi(-b);
  }
  return TQ_OK;
}

}  // namespace tq
