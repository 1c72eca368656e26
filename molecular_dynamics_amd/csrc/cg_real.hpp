// Real Clebsch-Gordan coupling tensors for l <= 2, built at compile time.
//
// "Unlocking Tensor Core Performance: GPU Acceleration for Machine Learning
// Interatomic Potentials" (section "Why MLIPs Need Dedicated Performance
// Optimization"): equivariant layers couple angular-momentum channels through
// Clebsch-Gordan coefficients.  The library builds them itself, independently
// of any table elsewhere:
//   1. complex coefficients <l1 m1 l2 m2 | l3 m3> by Racah's closed formula
//      (Condon-Shortley phase);
//   2. change to the real harmonic basis Y_lm (m = -l..l; l = 1 ordered
//      y, z, x): with U the complex->real unitary,
//      T[m1,m2,m3] = sum U1[m1,mu1] U2[m2,mu2] conj(U3[m3,mu3]) <..|..>,
//      which is purely real or purely imaginary; the nonzero part is kept;
//   3. scaled so that sum_{m1,m2} C[m1,m2,m3] C[m1,m2,m3'] = delta(m3,m3'),
//      sign fixed so the first nonzero entry (lexicographic m1, m2, m3) is > 0.
// Paths are all (l1, l2, l3) with |l1 - l2| <= l3 <= l1 + l2, lexicographic.
// Kernels iterate the nonzero lists with compile-time trip counts, so zero
// coefficients never reach the instruction stream.
#pragma once
#include <stdint.h>

namespace mdmp {
namespace cgc {

constexpr double csqrt(double x) {
  if (x <= 0) return 0.0;
  double g = x > 1 ? x : 1.0;
  for (int i = 0; i < 100; ++i) g = 0.5 * (g + x / g);
  return g;
}
constexpr double fact(int n) {
  double r = 1;
  for (int i = 2; i <= n; ++i) r *= i;
  return r;
}
constexpr double cabs(double x) { return x < 0 ? -x : x; }

// Racah's formula for <l1 m1 l2 m2 | l3 m3>
constexpr double cg_complex(int l1, int m1, int l2, int m2, int l3, int m3) {
  if (m1 + m2 != m3) return 0.0;
  if (l3 < (l1 > l2 ? l1 - l2 : l2 - l1) || l3 > l1 + l2) return 0.0;
  if (cabs(m1) > l1 || cabs(m2) > l2 || cabs(m3) > l3) return 0.0;
  double pre = csqrt((2 * l3 + 1) * fact(l3 + l1 - l2) * fact(l3 - l1 + l2) * fact(l1 + l2 - l3) /
                     fact(l1 + l2 + l3 + 1));
  double pre2 = csqrt(fact(l3 + m3) * fact(l3 - m3) * fact(l1 - m1) * fact(l1 + m1) * fact(l2 - m2) *
                      fact(l2 + m2));
  double s = 0;
  for (int k = 0; k <= l1 + l2 + l3; ++k) {
    int a[6] = {k, l1 + l2 - l3 - k, l1 - m1 - k, l2 + m2 - k, l3 - l2 + m1 + k, l3 - l1 - m2 + k};
    bool ok = true;
    for (int q = 0; q < 6; ++q) ok = ok && a[q] >= 0;
    if (!ok) continue;
    double den = 1;
    for (int q = 0; q < 6; ++q) den *= fact(a[q]);
    s += ((k & 1) ? -1.0 : 1.0) / den;
  }
  return pre * pre2 * s;
}

struct cplx {
  double re, im;
};
constexpr cplx cmul(cplx a, cplx b) { return {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re}; }
constexpr cplx cconj(cplx a) { return {a.re, -a.im}; }

// U[m][mu]: real harmonic Y_lm = sum_mu U[m][mu] Y_l^mu (complex, Condon-Shortley)
constexpr cplx umat(int m, int mu) {
  const double h = 0.70710678118654752440;
  if (m == 0) return {mu == 0 ? 1.0 : 0.0, 0.0};
  if (m > 0) {
    if (mu == m) return {(m & 1) ? -h : h, 0.0};
    if (mu == -m) return {h, 0.0};
    return {0.0, 0.0};
  }
  int a = -m;
  if (mu == -a) return {0.0, h};
  if (mu == a) return {0.0, (a & 1) ? h : -h};
  return {0.0, 0.0};
}

constexpr int kMaxL = 2;
constexpr int kMaxNnz = 32;

struct Path {
  int l1, l2, l3;
  int nnz;
  int8_t m1[kMaxNnz], m2[kMaxNnz], m3[kMaxNnz];  // 0..2l indices
  double v[kMaxNnz];
};

struct Table {
  int lmax, npaths, total_nnz;
  Path p[15];
};

constexpr Path make_path(int l1, int l2, int l3) {
  double re[5][5][5] = {}, im[5][5][5] = {};
  double nre = 0, nim = 0;
  for (int a = 0; a < 2 * l1 + 1; ++a)
    for (int b = 0; b < 2 * l2 + 1; ++b)
      for (int c = 0; c < 2 * l3 + 1; ++c) {
        cplx acc{0, 0};
        for (int u1 = -l1; u1 <= l1; ++u1)
          for (int u2 = -l2; u2 <= l2; ++u2) {
            int u3 = u1 + u2;
            if (u3 < -l3 || u3 > l3) continue;
            double cc = cg_complex(l1, u1, l2, u2, l3, u3);
            if (cc == 0) continue;
            cplx t = cmul(cmul(umat(a - l1, u1), umat(b - l2, u2)), cconj(umat(c - l3, u3)));
            acc.re += t.re * cc;
            acc.im += t.im * cc;
          }
        re[a][b][c] = acc.re;
        im[a][b][c] = acc.im;
        nre += acc.re * acc.re;
        nim += acc.im * acc.im;
      }
  bool use_im = nim > nre;
  double norm2 = use_im ? nim : nre;
  double scale = csqrt((2 * l3 + 1) / norm2);
  Path P{};
  P.l1 = l1;
  P.l2 = l2;
  P.l3 = l3;
  double sign = 0;
  for (int a = 0; a < 2 * l1 + 1; ++a)
    for (int b = 0; b < 2 * l2 + 1; ++b)
      for (int c = 0; c < 2 * l3 + 1; ++c) {
        double x = (use_im ? im[a][b][c] : re[a][b][c]) * scale;
        if (cabs(x) < 1e-12) continue;
        if (sign == 0) sign = x > 0 ? 1.0 : -1.0;
        P.m1[P.nnz] = (int8_t)a;
        P.m2[P.nnz] = (int8_t)b;
        P.m3[P.nnz] = (int8_t)c;
        P.v[P.nnz] = x * sign;
        P.nnz++;
      }
  return P;
}

constexpr Table make_table(int lmax) {
  Table t{};
  t.lmax = lmax;
  for (int a = 0; a <= lmax; ++a)
    for (int b = 0; b <= lmax; ++b)
      for (int c = 0; c <= lmax; ++c)
        if (c >= (a > b ? a - b : b - a) && c <= a + b) {
          t.p[t.npaths] = make_path(a, b, c);
          t.total_nnz += t.p[t.npaths].nnz;
          t.npaths++;
        }
  return t;
}

constexpr Table kTable1 = make_table(1);
constexpr Table kTable2 = make_table(2);

template <int L>
struct TableOf;
template <>
struct TableOf<1> {
  static constexpr const Table& t = kTable1;
};
template <>
struct TableOf<2> {
  static constexpr const Table& t = kTable2;
};

static_assert(kTable1.npaths == 5, "l<=1 has 5 paths");
static_assert(kTable2.npaths == 15, "l<=2 has 15 paths");

}  // namespace cgc
}  // namespace mdmp
