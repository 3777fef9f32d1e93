// The so(3) generators of the real Wigner-D blocks as a compile-time table.
//
// G_k^(l) = d/dt D^(l)(exp(t [e_k]_x)) at t = 0 (k = x, y, z; degree l block
// at gen_off(l), (2l+1)^2 entries row-major), evaluated with dual numbers
// a + b eps through the Ivanic-Ruedenberg recursion of the edge-frame rows:
// D^(l)(I + eps [e_k]_x) = I + eps G_k^(l) exactly, so the eps parts are the
// generators. The recursion and its coefficients are those of wig_entry in
// wigner.hpp, written here in constexpr form (square roots by Newton's
// iteration in double, then rounded to float like the host table).
//
// The torque and rotation-rate products of the kernels index this table with
// indices that are constants after unrolling, so its entries become literal
// operands instead of per-use memory reads.
#pragma once
#include "layout.hpp"

namespace so2 {
namespace gen_detail {

// square root of x >= 0 to double precision: Newton's iteration from above
constexpr double csqrt(double x) {
  if (x <= 0.0) return 0.0;
  double r = x > 1.0 ? x : 1.0;
  for (int i = 0; i < 200; ++i) {
    const double n = 0.5 * (r + x / r);
    if (n >= r) break;
    r = n;
  }
  return r;
}

struct Dual {
  double a = 0.0, b = 0.0;   // a + b eps, eps^2 = 0
};
constexpr Dual operator+(Dual x, Dual y) { return {x.a + y.a, x.b + y.b}; }
constexpr Dual operator-(Dual x, Dual y) { return {x.a - y.a, x.b - y.b}; }
constexpr Dual operator*(Dual x, Dual y) { return {x.a * y.a, x.a * y.b + x.b * y.a}; }
constexpr Dual scale(double s, Dual x) { return {s * x.a, s * x.b}; }

constexpr int kW = 2 * kMaxL + 1;
struct Level {
  Dual d[kW * kW];   // rows and columns -l..l of one degree, row-major, stride 2l + 1
};

// one P term: D1 row i (of -1, 0, 1) against row a of the previous degree
constexpr Dual wig_P(int i, int a, int b, int l, const Dual (&D1)[9], const Level& prev) {
  const int w = 2 * l - 1, rp = l - 1;
  const Dual* row = prev.d + (a + rp) * w + (l - 1);
  const Dual* r1 = D1 + (i + 1) * 3;
  if (b == l) return r1[2] * row[l - 1] - r1[0] * row[-(l - 1)];
  if (b == -l) return r1[2] * row[-(l - 1)] + r1[0] * row[l - 1];
  return r1[1] * row[b];
}

constexpr Dual wig_entry(int l, int m, int n, const Dual (&D1)[9], const Level& prev) {
  const int am = iabs(m);
  const double den = (n > -l && n < l) ? double((l + n) * (l - n)) : double((2 * l) * (2 * l - 1));
  Dual out;
  if (am < l) out = out + scale(csqrt(double((l + m) * (l - m)) / den), wig_P(0, m, n, l, D1, prev));
  {
    const double v = (m == 0 ? -0.5 : 0.5) * csqrt(double((m == 0 ? 2 : 1) * (l + am - 1) * (l + am)) / den);
    Dual V;
    if (m == 0) V = wig_P(1, 1, n, l, D1, prev) + wig_P(-1, -1, n, l, D1, prev);
    else if (m > 0)
      V = (m == 1) ? scale(1.4142135623730951, wig_P(1, 0, n, l, D1, prev))
                   : wig_P(1, m - 1, n, l, D1, prev) - wig_P(-1, -m + 1, n, l, D1, prev);
    else
      V = (m == -1) ? scale(1.4142135623730951, wig_P(-1, 0, n, l, D1, prev))
                    : wig_P(1, m + 1, n, l, D1, prev) + wig_P(-1, -m - 1, n, l, D1, prev);
    out = out + scale(v, V);
  }
  if (m != 0 && am <= l - 2) {
    const double w = -0.5 * csqrt(double((l - am - 1) * (l - am)) / den);
    const Dual W = (m > 0) ? wig_P(1, m + 1, n, l, D1, prev) + wig_P(-1, -m - 1, n, l, D1, prev)
                           : wig_P(1, m - 1, n, l, D1, prev) - wig_P(-1, -m + 1, n, l, D1, prev);
    out = out + scale(w, W);
  }
  return out;
}

}  // namespace gen_detail

struct GenTable {
  float v[3 * kGenSize];
};

constexpr GenTable make_gen_table() {
  using gen_detail::Dual;
  using gen_detail::Level;
  GenTable t{};
  // [e_k]_x, row-major
  const int cross[3][9] = {{0, 0, 0, 0, 0, -1, 0, 1, 0}, {0, 0, 1, 0, 0, 0, -1, 0, 0}, {0, -1, 0, 1, 0, 0, 0, 0, 0}};
  const int p[3] = {1, 2, 0};   // D^(1) in the (y, z, x) component order
  for (int k = 0; k < 3; ++k) {
    Dual R[9] = {};
    for (int a = 0; a < 9; ++a) R[a] = Dual{(a % 4 == 0) ? 1.0 : 0.0, double(cross[k][a])};
    Dual D1[9] = {};
    for (int a = 0; a < 3; ++a)
      for (int b = 0; b < 3; ++b) D1[a * 3 + b] = R[p[a] * 3 + p[b]];
    float* G = t.v + k * kGenSize;
    for (int a = 0; a < 9; ++a) G[gen_off(1) + a] = float(D1[a].b);
    Level prev{}, cur{};
    for (int a = 0; a < 9; ++a) prev.d[a] = D1[a];
    for (int l = 2; l <= kMaxL; ++l) {
      const int n = 2 * l + 1;
      for (int m = -l; m <= l; ++m)
        for (int c = -l; c <= l; ++c) cur.d[(m + l) * n + c + l] = gen_detail::wig_entry(l, m, c, D1, prev);
      for (int a = 0; a < n * n; ++a) G[gen_off(l) + a] = float(cur.d[a].b);
      prev = cur;
    }
  }
  return t;
}

}  // namespace so2
