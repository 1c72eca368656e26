// Device-side building blocks shared by the model kernels.
#pragma once
#include "cg_real.hpp"
#include "common.hpp"

namespace mdmp {

// per active edge geometry record (float32), stride kGeo
constexpr int kGeo = 24;
constexpr int G_R = 0, G_U = 1, G_DU = 2, G_RH = 3, G_B = 6, G_Y = 14;
constexpr int kNB = 8;    // Bessel functions
constexpr int kHR = 64;   // radial hidden width
constexpr int kTE = 16;   // edges per MFMA tile
constexpr int kNW = 4;    // waves per block in the edge kernels

typedef float f4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
typedef short s8v __attribute__((ext_vector_type(8)));

template <int L>
struct Dims {
  static constexpr int K = (L + 1) * (L + 1);
  static constexpr int NP = cgc::TableOf<L>::t.npaths;
};

// orthonormal real spherical harmonics of a unit vector (m = -l..l; l=1 is y, z, x)
template <int L>
__device__ __forceinline__ void real_sh(float x, float y, float z, float* Y) {
  Y[0] = 0.28209479177387814f;
  if (L >= 1) {
    const float c1 = 0.4886025119029199f;
    Y[1] = c1 * y;
    Y[2] = c1 * z;
    Y[3] = c1 * x;
  }
  if (L >= 2) {
    const float a = 1.0925484305920792f, b = 0.31539156525252005f, c = 0.5462742152960396f;
    Y[4] = a * x * y;
    Y[5] = a * y * z;
    Y[6] = b * (3.0f * z * z - 1.0f);
    Y[7] = a * x * z;
    Y[8] = c * (x * x - y * y);
  }
}

// gradient of the harmonic polynomials w.r.t. (x, y, z), contracted with g[K]
template <int L>
__device__ __forceinline__ void real_sh_grad(float x, float y, float z, const float* g, float& gx, float& gy,
                                             float& gz) {
  gx = gy = gz = 0.f;
  if (L >= 1) {
    const float c1 = 0.4886025119029199f;
    gy += c1 * g[1];
    gz += c1 * g[2];
    gx += c1 * g[3];
  }
  if (L >= 2) {
    const float a = 1.0925484305920792f, b = 0.31539156525252005f, c = 0.5462742152960396f;
    gx += a * y * g[4];
    gy += a * x * g[4];
    gy += a * z * g[5];
    gz += a * y * g[5];
    gz += b * 6.0f * z * g[6];
    gx += a * z * g[7];
    gz += a * x * g[7];
    gx += c * 2.0f * x * g[8];
    gy -= c * 2.0f * y * g[8];
  }
}

// edge vector d = x_j - x_i with d -= L * rint(d / L), float32, no contraction
__device__ __forceinline__ void edge_vec(const float* __restrict__ pos, int i, int j, float L, float inv_L,
                                         float& dx, float& dy, float& dz) {
#pragma clang fp contract(off)
  dx = pos[3 * j + 0] - pos[3 * i + 0];
  dy = pos[3 * j + 1] - pos[3 * i + 1];
  dz = pos[3 * j + 2] - pos[3 * i + 2];
  float sx = L * rintf(dx * inv_L);
  float sy = L * rintf(dy * inv_L);
  float sz = L * rintf(dz * inv_L);
  dx = dx - sx;
  dy = dy - sy;
  dz = dz - sz;
}

__device__ __forceinline__ float edge_r(float dx, float dy, float dz) {
#pragma clang fp contract(off)
  float a = dx * dx;
  float b = dy * dy;
  float c = dz * dz;
  return sqrtf((a + b) + c);
}

// Tensor product v^{l3}[m3] += w_p sum CG_p[m1,m2,m3] x^{l1}[m1] Y^{l2}[m2], all paths
template <int L>
__device__ __forceinline__ void tp_fwd(const float* x, const float* Y, const float* w, float* v) {
  constexpr const cgc::Table& T = cgc::TableOf<L>::t;
#pragma unroll
  for (int p = 0; p < T.npaths; ++p) {
    const int l1 = T.p[p].l1, l2 = T.p[p].l2, l3 = T.p[p].l3;
    float G[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int z = 0; z < T.p[p].nnz; ++z)
      G[T.p[p].m3[z]] += (float)T.p[p].v[z] * (x[l1 * l1 + T.p[p].m1[z]] * Y[l2 * l2 + T.p[p].m2[z]]);
#pragma unroll
    for (int m = 0; m < 2 * l3 + 1; ++m) v[l3 * l3 + m] += w[p] * G[m];
  }
}

// Same product keeping every path's G_p (for the backward): G laid out path-major
template <int L>
struct GOff {
  static constexpr int total() {
    int s = 0;
    for (int p = 0; p < cgc::TableOf<L>::t.npaths; ++p) s += 2 * cgc::TableOf<L>::t.p[p].l3 + 1;
    return s;
  }
  static constexpr int off(int q) {
    int s = 0;
    for (int p = 0; p < q; ++p) s += 2 * cgc::TableOf<L>::t.p[p].l3 + 1;
    return s;
  }
};

template <int L>
__device__ __forceinline__ void tp_fwd_keep(const float* x, const float* Y, const float* w, float* v,
                                            float* G) {
  constexpr const cgc::Table& T = cgc::TableOf<L>::t;
#pragma unroll
  for (int p = 0; p < T.npaths; ++p) {
    const int l1 = T.p[p].l1, l2 = T.p[p].l2, l3 = T.p[p].l3;
    float* Gp = G + GOff<L>::off(p);
#pragma unroll
    for (int m = 0; m < 2 * l3 + 1; ++m) Gp[m] = 0.f;
#pragma unroll
    for (int z = 0; z < T.p[p].nnz; ++z)
      Gp[T.p[p].m3[z]] += (float)T.p[p].v[z] * (x[l1 * l1 + T.p[p].m1[z]] * Y[l2 * l2 + T.p[p].m2[z]]);
#pragma unroll
    for (int m = 0; m < 2 * l3 + 1; ++m) v[l3 * l3 + m] += w[p] * Gp[m];
  }
}

// t^{l2}[m2] += sum_p sum CG_p[m1,m2,m3] x^{l1}[m1] wg_p^{l3}[m3]   (gradient w.r.t. Y)
// wg_p = w_p * gv^{l3}
template <int L>
__device__ __forceinline__ void tp_grad_y(const float* x, const float* gv, const float* w, float* t) {
  constexpr const cgc::Table& T = cgc::TableOf<L>::t;
#pragma unroll
  for (int p = 0; p < T.npaths; ++p) {
    const int l1 = T.p[p].l1, l2 = T.p[p].l2, l3 = T.p[p].l3;
    float wg[5];
#pragma unroll
    for (int m = 0; m < 2 * l3 + 1; ++m) wg[m] = w[p] * gv[l3 * l3 + m];
#pragma unroll
    for (int z = 0; z < T.p[p].nnz; ++z)
      t[l2 * l2 + T.p[p].m2[z]] += (float)T.p[p].v[z] * (x[l1 * l1 + T.p[p].m1[z]] * wg[T.p[p].m3[z]]);
  }
}

// gx^{l1}[m1] += sum_p sum CG_p[m1,m2,m3] Y^{l2}[m2] w_p gv^{l3}[m3]   (gradient w.r.t. x)
template <int L>
__device__ __forceinline__ void tp_grad_x(const float* Y, const float* gv, const float* w, float* gx) {
  constexpr const cgc::Table& T = cgc::TableOf<L>::t;
#pragma unroll
  for (int p = 0; p < T.npaths; ++p) {
    const int l1 = T.p[p].l1, l2 = T.p[p].l2, l3 = T.p[p].l3;
    float wg[5];
#pragma unroll
    for (int m = 0; m < 2 * l3 + 1; ++m) wg[m] = w[p] * gv[l3 * l3 + m];
#pragma unroll
    for (int z = 0; z < T.p[p].nnz; ++z)
      gx[l1 * l1 + T.p[p].m1[z]] += (float)T.p[p].v[z] * (Y[l2 * l2 + T.p[p].m2[z]] * wg[T.p[p].m3[z]]);
  }
}

__device__ __forceinline__ float group_sum_rt(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace mdmp
