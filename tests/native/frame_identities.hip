#include "kernels.hpp"
#include <cstdio>
#include <random>
#include <cmath>
using namespace mdmp;
template <int L> double run(std::mt19937& rng, float rx, float ry, float rz) {
  constexpr int K = Dims<L>::K, NP = Dims<L>::NP;
  std::normal_distribution<float> nd;
  float x[K], w[NP], gm[K], gv[K];
  for (int k = 0; k < K; ++k) { x[k] = nd(rng); gm[k] = nd(rng); gv[k] = nd(rng); }
  for (int p = 0; p < NP; ++p) w[p] = nd(rng);
  float Y[K]; real_sh<L>(rx, ry, rz, Y);
  float R[9]; edge_frame(rx, ry, rz, R);
  float d2[25] = {0};
  if (L >= 2) for (int m = 0; m < 5; ++m) wigner2_row(R, m, d2 + 5 * m);
  double err = 0;
  // Y(R v) = D Y(v) for a random v
  { float v[3] = {nd(rng), nd(rng), nd(rng)}; float n = std::sqrt(v[0]*v[0]+v[1]*v[1]+v[2]*v[2]); for (auto& a : v) a /= n;
    float u[3]; for (int a = 0; a < 3; ++a) u[a] = R[3*a]*v[0] + R[3*a+1]*v[1] + R[3*a+2]*v[2];
    float Yv[K], Yu[K], DY[K]; real_sh<L>(v[0], v[1], v[2], Yv); real_sh<L>(u[0], u[1], u[2], Yu);
    rot_in<L>(R, d2, Yv, DY);
    for (int k = 0; k < K; ++k) err = std::max(err, (double)std::fabs(DY[k] - Yu[k]));
    // R rhat = z
    float Yz[K]; rot_in<L>(R, d2, Y, Yz);
    float Yp[K]; real_sh<L>(0.f, 0.f, 1.f, Yp);
    for (int k = 0; k < K; ++k) err = std::max(err, (double)std::fabs(Yz[k] - Yp[k]));
  }
  // forward
  { float v[K] = {0}, xp[K], vp[K] = {0}, v2[K] = {0};
    tp_fwd<L, 0>(x, Y, w, v); rot_in<L>(R, d2, x, xp); tpz_fwd<L>(xp, w, vp); rot_out_add<L>(R, d2, vp, v2);
    for (int k = 0; k < K; ++k) err = std::max(err, (double)std::fabs(v[k] - v2[k])); }
  // dot / y0
  { float dot[NP], y0[NP], dot2[NP], y02[NP], xp[K], gmp[K];
    tp_fwd_dot<L, 0, K>(x, Y, gm, dot, y0); rot_in<L>(R, d2, x, xp); rot_in<L>(R, d2, gm, gmp); tpz_fwd_dot<L>(xp, gmp, dot2, y02);
    for (int p = 0; p < NP; ++p) err = std::max(err, (double)std::max(std::fabs(dot[p] - dot2[p]), std::fabs(y0[p] - y02[p]))); }
  // tangential gradient
  { float t[K] = {0}; tp_grad_y<L, 0>(x, gv, w, t); float g[3]; real_sh_grad<L>(rx, ry, rz, t, g[0], g[1], g[2]);
    float dt = rx*g[0] + ry*g[1] + rz*g[2]; float r[3] = {rx, ry, rz};
    float xp[K], gvp[K]; rot_in<L>(R, d2, x, xp); rot_in<L>(R, d2, gv, gvp);
    float gx = 0, gy = 0; tpz_grad_dir<L>(xp, gvp, w, gx, gy);
    for (int q = 0; q < 3; ++q) err = std::max(err, (double)std::fabs((g[q] - dt * r[q]) - (gx * R[q] + gy * R[3 + q]))); }
  // input gradient, edge seen from the other end (direction -rhat in the frame)
  { float Ye[K]; real_sh<L>(-rx, -ry, -rz, Ye);
    float gl[K] = {0}; tp_grad_x<L, 0>(Ye, gv, w, gl);
    float gvp[K], gxp[K] = {0}, g2[K] = {0}; rot_in<L>(R, d2, gv, gvp); tpz_grad_x<L, true>(gvp, w, gxp); rot_out_add<L>(R, d2, gxp, g2);
    for (int k = 0; k < K; ++k) err = std::max(err, (double)std::fabs(gl[k] - g2[k])); }
  return err;
}
int main() {
  // lab-frame products (kernels.hpp) against their edge-frame forms, fp32, random directions and both poles
  std::mt19937 rng(3); std::normal_distribution<float> nd;
  double e1 = 0, e2 = 0;
  for (int it = 0; it < 20000; ++it) {
    float v[3] = {nd(rng), nd(rng), nd(rng)};
    if (it % 5 == 0) { v[0] *= 0.01f; v[1] *= 0.01f; }
    if (it == 7) { v[0] = 0; v[1] = 0; v[2] = 1; }
    if (it == 8) { v[0] = 0; v[1] = 0; v[2] = -1; }
    if (it == 9) { v[0] = 1; v[1] = 0; v[2] = 0; }
    float n = std::sqrt(v[0]*v[0]+v[1]*v[1]+v[2]*v[2]);
    e1 = std::max(e1, run<1>(rng, v[0]/n, v[1]/n, v[2]/n));
    e2 = std::max(e2, run<2>(rng, v[0]/n, v[1]/n, v[2]/n));
  }
  printf("max abs err l<=1 %.3e  l<=2 %.3e\n", e1, e2);
  return (e1 < 1e-4 && e2 < 1e-4) ? 0 : 1;
}
