// Device-side building blocks shared by the model kernels.
#pragma once
#include "cg_real.hpp"
#include "common.hpp"

namespace mdmp {

// Per active edge geometry (float32).  The record in HBM (stride kGeoH) holds r, u,
// du/dr, rhat[3], B[8] and two zero words; the tile's copy in LDS (stride kGeo) adds
// at G_Y the harmonics Y[K] of rhat (lab-frame layers) or the rows of the edge's
// rotation (edge-frame layers), both formed from rhat when the tile is loaded.
constexpr int kGeo = 24;
constexpr int kGeoH = 16;
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
__host__ __device__ __forceinline__ void real_sh(float x, float y, float z, float* Y) {
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
__host__ __device__ __forceinline__ void real_sh_grad(float x, float y, float z, const float* g, float& gx, float& gy,
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

// minimum image of a difference vector: d -= L * rint(d / L), float32, no contraction
__device__ __forceinline__ void min_image(float x, float y, float z, float L, float inv_L, float& dx, float& dy,
                                          float& dz) {
#pragma clang fp contract(off)
  float sx = L * rintf(x * inv_L);
  float sy = L * rintf(y * inv_L);
  float sz = L * rintf(z * inv_L);
  dx = x - sx;
  dy = y - sy;
  dz = z - sz;
}

// edge vector d = x_j - x_i, minimum image
__device__ __forceinline__ void edge_vec(const float* __restrict__ pos, int i, int j, float L, float inv_L,
                                         float& dx, float& dy, float& dz) {
  min_image(pos[3 * j + 0] - pos[3 * i + 0], pos[3 * j + 1] - pos[3 * i + 1], pos[3 * j + 2] - pos[3 * i + 2], L,
            inv_L, dx, dy, dz);
}

__device__ __forceinline__ float edge_r(float dx, float dy, float dz) {
#pragma clang fp contract(off)
  float a = dx * dx;
  float b = dy * dy;
  float c = dz * dz;
  return sqrtf((a + b) + c);
}

// ---------------------------------------------------------------- path sets
// MODE bit 1: only paths with l1 = 0 (first layer: every input with l > 0 is
// exactly zero); MODE bit 2: only paths with l3 = 0 (last layer: only the
// scalar channel reaches the energy).  Paths are in lexicographic order, so
// the l1 = 0 paths come first and the l3 = 0 paths are (l, l, 0).
template <int L, int MODE>
struct Paths {
  static constexpr bool on(int p) {
    return !((MODE & 1) && cgc::TableOf<L>::t.p[p].l1 != 0) && !((MODE & 2) && cgc::TableOf<L>::t.p[p].l3 != 0);
  }
  static constexpr int count() {
    int n = 0;
    for (int p = 0; p < cgc::TableOf<L>::t.npaths; ++p) n += on(p) ? 1 : 0;
    return n;
  }
  static constexpr int idx(int q) {
    for (int p = 0; p < cgc::TableOf<L>::t.npaths; ++p)
      if (on(p) && q-- == 0) return p;
    return -1;
  }
};

// runtime path index of the q-th active path (the same mapping as Paths::idx)
template <int L, int MODE>
__device__ __forceinline__ int path_of(int q) {
  if constexpr (MODE == 0 || MODE == 1) return q;
  else if constexpr (MODE == 3) return 0;
  else if constexpr (L == 1) return q == 0 ? 0 : 3;
  else return q == 0 ? 0 : (q == 1 ? 4 : 12);
}
static_assert(Paths<2, 2>::idx(1) == 4 && Paths<2, 2>::idx(2) == 12 && Paths<1, 2>::idx(1) == 3, "path map");
static_assert(Paths<2, 1>::idx(2) == 2 && Paths<2, 1>::count() == 3 && Paths<2, 3>::count() == 1, "path map");

// Tensor product over the active paths q (w indexed by q):
// v^{l3}[m3] += w_q sum CG_p[m1,m2,m3] x^{l1}[m1] Y^{l2}[m2]
template <int L, int MODE>
__host__ __device__ __forceinline__ void tp_fwd(const float* x, const float* Y, const float* w, float* v) {
  constexpr const cgc::Table& T = cgc::TableOf<L>::t;
#pragma unroll
  for (int q = 0; q < Paths<L, MODE>::count(); ++q) {
    const int p = Paths<L, MODE>::idx(q);
    const int l1 = T.p[p].l1, l2 = T.p[p].l2, l3 = T.p[p].l3;
    float G[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int z = 0; z < T.p[p].nnz; ++z)
      G[T.p[p].m3[z]] += (float)T.p[p].v[z] * (x[l1 * l1 + T.p[p].m1[z]] * Y[l2 * l2 + T.p[p].m2[z]]);
#pragma unroll
    for (int m = 0; m < 2 * l3 + 1; ++m) v[l3 * l3 + m] += w[q] * G[m];
  }
}

// Forward product contracted with a fixed vector gm: for every active path q the
// output y_q[m3] = sum CG_p[m1,m2,m3] x^{l1}[m1] Y^{l2}[m2] is formed and only
// dot[q] = sum_m3 gm^{l3}[m3] y_q[m3] (components at or past KV skipped) and, for
// l3 = 0, y0[q] = y_q[0] are kept.  With v = sum_q w_q y_q this gives gm . v =
// sum_q w_q dot[q], v^0 = sum_{q: l3 = 0} w_q y0[q] and dE/dw_q without storing v or y.
template <int L, int MODE, int KV>
__host__ __device__ __forceinline__ void tp_fwd_dot(const float* x, const float* Y, const float* gm, float* dot, float* y0) {
  constexpr const cgc::Table& T = cgc::TableOf<L>::t;
#pragma unroll
  for (int q = 0; q < Paths<L, MODE>::count(); ++q) {
    const int p = Paths<L, MODE>::idx(q);
    const int l1 = T.p[p].l1, l2 = T.p[p].l2, l3 = T.p[p].l3;
    float G[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int z = 0; z < T.p[p].nnz; ++z)
      G[T.p[p].m3[z]] += (float)T.p[p].v[z] * (x[l1 * l1 + T.p[p].m1[z]] * Y[l2 * l2 + T.p[p].m2[z]]);
    float d = 0.f;
#pragma unroll
    for (int m = 0; m < 2 * l3 + 1; ++m)
      if (l3 * l3 + m < KV) d += gm[l3 * l3 + m] * G[m];
    dot[q] = d;
    y0[q] = l3 == 0 ? G[0] : 0.f;
  }
}

// t^{l2}[m2] += sum_q w_q sum CG_p[m1,m2,m3] x^{l1}[m1] gv^{l3}[m3]     (dE/dY)
// The products x gv are shared by all paths; w_q is applied once per path output.
template <int L, int MODE>
__host__ __device__ __forceinline__ void tp_grad_y(const float* x, const float* gv, const float* w, float* t) {
  constexpr const cgc::Table& T = cgc::TableOf<L>::t;
#pragma unroll
  for (int q = 0; q < Paths<L, MODE>::count(); ++q) {
    const int p = Paths<L, MODE>::idx(q);
    const int l1 = T.p[p].l1, l2 = T.p[p].l2, l3 = T.p[p].l3;
    float acc[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int z = 0; z < T.p[p].nnz; ++z)
      acc[T.p[p].m2[z]] += (float)T.p[p].v[z] * (x[l1 * l1 + T.p[p].m1[z]] * gv[l3 * l3 + T.p[p].m3[z]]);
#pragma unroll
    for (int m = 0; m < 2 * l2 + 1; ++m) t[l2 * l2 + m] += w[q] * acc[m];
  }
}

// gx^{l1}[m1] += sum_q w_q sum CG_p[m1,m2,m3] Y^{l2}[m2] gv^{l3}[m3]      (dE/dht)
template <int L, int MODE>
__host__ __device__ __forceinline__ void tp_grad_x(const float* Y, const float* gv, const float* w, float* gx) {
  constexpr const cgc::Table& T = cgc::TableOf<L>::t;
#pragma unroll
  for (int q = 0; q < Paths<L, MODE>::count(); ++q) {
    const int p = Paths<L, MODE>::idx(q);
    const int l1 = T.p[p].l1, l2 = T.p[p].l2, l3 = T.p[p].l3;
    float acc[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int z = 0; z < T.p[p].nnz; ++z)
      acc[T.p[p].m1[z]] += (float)T.p[p].v[z] * (Y[l2 * l2 + T.p[p].m2[z]] * gv[l3 * l3 + T.p[p].m3[z]]);
#pragma unroll
    for (int m = 0; m < 2 * l1 + 1; ++m) gx[l1 * l1 + m] += w[q] * acc[m];
  }
}

// ---------------------------------------------------------------- row order over the XCDs
// Workgroups are handed to the 8 XCDs (each with its own L2) round-robin in launch
// order.  The edge kernels renumber their (row, channel block) grid so that each XCD
// walks chunks of kXcdChunk consecutive (row, channel block) pairs, the channel blocks
// of a row adjacent: the blocks of a row share its edges' geometry and sender indices,
// and Hilbert-sorted rows of a chunk share most of their neighbours, so both stay in
// that XCD's L2; chunks alternate between the XCDs, which balances dense and sparse
// regions.
constexpr int kXcdChunk = 512;
__device__ __forceinline__ void xcd_row_block(int& row, int& cb) {
  const int64_t nrow = gridDim.x, ncb = gridDim.y;
  const int64_t L = xcd_order(blockIdx.x + (int64_t)blockIdx.y * nrow, nrow * ncb, kXcdChunk);
  row = (int)(L / ncb);
  cb = (int)(L % ncb);
}

// ---------------------------------------------------------------- edge-aligned frame
// The coupling tensors are rotation invariant: CG(D x, D Y) = D CG(x, Y) for the
// real Wigner matrices D of any rotation (the equivariance of the layer, "Unlocking
// Tensor Core Performance", section "Why MLIPs Need Dedicated Performance
// Optimization").  With R the rotation that takes rhat to the pole z-hat, every
// harmonic of the pole vanishes except m = 0, so the product over the edge reduces
// to the entries with m2 = 0 (37 of 137 for l <= 2):
//   CG(x, Y(rhat)) = D^T CG(D x, Y(z-hat)).
// Gradients with respect to rhat need only the tangential derivatives at the pole,
// d/dx of Y_{l,+1} and d/dy of Y_{l,-1} (72 entries), rotated back with R^T.
// R has rows e1, e2, rhat; D on l = 1 is R with indices permuted to (y, z, x);
// D on l = 2 is stored per edge (25 values, computed by frame_setup).

// Y_l(z-hat) at m = 0, and d/dx Y_{l,+1} = d/dy Y_{l,-1} at z-hat (forms of real_sh)
__host__ __device__ constexpr double ypole(int l) {
  return l == 0 ? 0.28209479177387814 : (l == 1 ? 0.4886025119029199 : 2.0 * 0.31539156525252005);
}
__host__ __device__ constexpr double ydpole(int l) { return l == 1 ? 0.4886025119029199 : 1.0925484305920792; }
// component a of the l = 1 block (y, z, x) is Cartesian axis pi1(a)
__host__ __device__ constexpr int pi1(int a) { return a == 0 ? 1 : (a == 1 ? 2 : 0); }

// rows of R for a unit vector (x, y, z): e1 = normalize(a x rhat) with a = z-hat, or
// x-hat near the poles; e2 = rhat x e1.  Right-handed, R rhat = z-hat.
__host__ __device__ inline void edge_frame(float x, float y, float z, float* R) {
  float ax, ay, az;  // a x rhat
  if (fabsf(z) < 0.9f) {
    ax = -y; ay = x; az = 0.f;
  } else {
    ax = 0.f; ay = -z; az = y;
  }
  const float inv = 1.0f / sqrtf(ax * ax + ay * ay + az * az);
  ax *= inv; ay *= inv; az *= inv;
  R[0] = ax; R[1] = ay; R[2] = az;
  R[3] = y * az - z * ay; R[4] = z * ax - x * az; R[5] = x * ay - y * ax;
  R[6] = x; R[7] = y; R[8] = z;
}

// Row m of the l = 2 Wigner matrix of R (real harmonics xy, yz, 3z^2-1, xz, x^2-y^2
// with scales s = (a, a, b, a, c)): the quadratic form p_m(R v) = v^T S v is
// re-expanded in the p_n, and D[m][n] = s_m / s_n * coefficient.  With rows r0, r1,
// r2 of R: S = sym(r0 r1^T), sym(r1 r2^T), 2 r2 r2^T - r0 r0^T - r1 r1^T,
// sym(r0 r2^T), r0 r0^T - r1 r1^T for m = 0..4 (selected without branches).
__host__ __device__ inline void wigner2_row(const float* R, int m, float* row) {
  const bool sy = m == 0 || m == 1 || m == 3;  // symmetrised outer product
  const float* pa = m == 1 ? R + 3 : R;
  const float* pb = m == 0 ? R + 3 : R + 6;
  const float ca = sy ? 0.f : (m == 2 ? -1.f : 1.f);  // coefficient of r0 r0^T
  const float cb = sy ? 0.f : -1.f;                   // r1 r1^T
  const float cc = m == 2 ? 2.f : 0.f;                // r2 r2^T
  const float cs = sy ? 1.f : 0.f;
  float a[3], b[3];
  for (int i = 0; i < 3; ++i) {
    a[i] = pa[i];
    b[i] = pb[i];
  }
  auto S = [&](int i, int j) {
    return cs * 0.5f * (a[i] * b[j] + b[i] * a[j]) + ca * R[i] * R[j] + cb * R[3 + i] * R[3 + j] +
           cc * R[6 + i] * R[6 + j];
  };
  // s_m / s_n with the scales (a, a, b, a, c): a / b = 3.4641016, a / c = 2
  constexpr float ab = 3.4641016151377544f, ac = 2.0f;
  const float ra = (m == 2) ? 1.0f / ab : (m == 4 ? 1.0f / ac : 1.0f);  // s_m / a
  const float rb = (m == 2) ? 1.0f : (m == 4 ? ab / ac : ab);           // s_m / b
  const float rc = (m == 2) ? ac / ab : (m == 4 ? 1.0f : ac);           // s_m / c
  row[0] = ra * 2.0f * S(0, 1);
  row[1] = ra * 2.0f * S(1, 2);
  row[2] = rb * 0.5f * S(2, 2);
  row[3] = ra * 2.0f * S(0, 2);
  row[4] = rc * 0.5f * (S(0, 0) - S(1, 1));
}

constexpr int kD2 = 28;  // per-edge stride of the stored l = 2 blocks (25 used)

// Frames of a tile: R over the harmonic slots of the geometry record (they are not
// used in the frame) and the l = 2 blocks in d2[TE][kD2].  Padded edges get the
// frame of z-hat.  Ends with a barrier; d2 must be free when it is called.
template <int TE, bool OPAQUE = false>
__device__ __forceinline__ void frame_setup(float* s_geo, float* d2, int nv, int tid) {
  // OPAQUE: the thread's role (edge, row of D_2) and the constants it selects are rebuilt
  // here at every tile rather than hoisted out of the tile loop (where they spill in the
  // register-bound sender pass)
  if constexpr (OPAQUE) asm volatile("" : "+v"(tid));
  constexpr int TPE = 256 / TE;
  static_assert(TPE >= 6, "threads per edge");
  const int e = tid / TPE, k = tid % TPE;
  float* g = s_geo + e * kGeo;
  const bool on = e < nv;
  float R[9];
  edge_frame(on ? g[G_RH] : 0.f, on ? g[G_RH + 1] : 0.f, on ? g[G_RH + 2] : 1.f, R);
  if (k < 5) {
    float row[5];
    wigner2_row(R, k, row);
#pragma unroll
    for (int n = 0; n < 5; ++n) d2[e * kD2 + 5 * k + n] = row[n];
  } else if (k == 5) {
#pragma unroll
    for (int n = 0; n < 9; ++n) g[G_Y + n] = R[n];
  }
  __syncthreads();
}

// x' = D x on the blocks l = 1..L (l = 0 is unchanged)
template <int L>
__host__ __device__ __forceinline__ void rot_in(const float* R, const float* d2, const float* x, float* xp) {
  xp[0] = x[0];
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    float s = 0.f;
#pragma unroll
    for (int b = 0; b < 3; ++b) s += R[3 * pi1(a) + pi1(b)] * x[1 + b];
    xp[1 + a] = s;
  }
  if constexpr (L >= 2) {
#pragma unroll
    for (int m = 0; m < 5; ++m) {
      float s = 0.f;
#pragma unroll
      for (int n = 0; n < 5; ++n) s += d2[5 * m + n] * x[4 + n];
      xp[4 + m] = s;
    }
  }
}

// out += D^T y
template <int L>
__host__ __device__ __forceinline__ void rot_out_add(const float* R, const float* d2, const float* y, float* out) {
  out[0] += y[0];
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    float s = 0.f;
#pragma unroll
    for (int a = 0; a < 3; ++a) s += R[3 * pi1(a) + pi1(b)] * y[1 + a];
    out[1 + b] += s;
  }
  if constexpr (L >= 2) {
#pragma unroll
    for (int n = 0; n < 5; ++n) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < 5; ++m) s += d2[5 * m + n] * y[4 + m];
      out[4 + n] += s;
    }
  }
}

// does path p have an entry with m2 = M2 and m3 (or m1, when BY_M1) = M?
template <int L>
constexpr bool pole_touch(int p, int M2, int M, bool by_m1) {
  const cgc::Path& P = cgc::TableOf<L>::t.p[p];
  for (int z = 0; z < P.nnz; ++z)
    if (P.m2[z] == M2 && (by_m1 ? P.m1[z] : P.m3[z]) == M) return true;
  return false;
}

// v'^{l3}[m3] += w_p sum_{m1} CG_p[m1, 0, m3] Y_{l2}(z-hat) x'^{l1}[m1]   (all paths)
template <int L>
__host__ __device__ __forceinline__ void tpz_fwd(const float* xp, const float* w, float* vp) {
  constexpr const cgc::Table& T = cgc::TableOf<L>::t;
#pragma unroll
  for (int p = 0; p < T.npaths; ++p) {
    const int l1 = T.p[p].l1, l2 = T.p[p].l2, l3 = T.p[p].l3;
    float G[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int z = 0; z < T.p[p].nnz; ++z)
      if (T.p[p].m2[z] == l2) G[T.p[p].m3[z]] += (float)(T.p[p].v[z] * ypole(l2)) * xp[l1 * l1 + T.p[p].m1[z]];
#pragma unroll
    for (int m = 0; m < 2 * l3 + 1; ++m)
      if (pole_touch<L>(p, l2, m, false)) vp[l3 * l3 + m] += w[p] * G[m];
  }
}

// dot[p] = gm' . y'_p and y0[p] = y'_p[0] (l3 = 0) of the pole products y'_p
template <int L>
__host__ __device__ __forceinline__ void tpz_fwd_dot(const float* xp, const float* gmp, float* dot, float* y0) {
  constexpr const cgc::Table& T = cgc::TableOf<L>::t;
#pragma unroll
  for (int p = 0; p < T.npaths; ++p) {
    const int l1 = T.p[p].l1, l2 = T.p[p].l2, l3 = T.p[p].l3;
    float G[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int z = 0; z < T.p[p].nnz; ++z)
      if (T.p[p].m2[z] == l2) G[T.p[p].m3[z]] += (float)(T.p[p].v[z] * ypole(l2)) * xp[l1 * l1 + T.p[p].m1[z]];
    float d = 0.f;
#pragma unroll
    for (int m = 0; m < 2 * l3 + 1; ++m)
      if (pole_touch<L>(p, l2, m, false)) d += gmp[l3 * l3 + m] * G[m];
    dot[p] = d;
    y0[p] = l3 == 0 ? G[0] : 0.f;
  }
}

// tangential gradient at the pole: gx = sum_p w_p sum CG_p[m1, +1, m3] dY x'[m1] gv'[m3],
// gy the same with m2 = -1 (components along e1 and e2 of dE/drhat)
template <int L>
__host__ __device__ __forceinline__ void tpz_grad_dir(const float* xp, const float* gvp, const float* w, float& gx,
                                             float& gy) {
  constexpr const cgc::Table& T = cgc::TableOf<L>::t;
#pragma unroll
  for (int p = 0; p < T.npaths; ++p) {
    const int l1 = T.p[p].l1, l2 = T.p[p].l2, l3 = T.p[p].l3;
    if (l2 == 0) continue;
    float ax = 0.f, ay = 0.f;
#pragma unroll
    for (int z = 0; z < T.p[p].nnz; ++z) {
      const float cf = (float)(T.p[p].v[z] * ydpole(l2));
      const float pr = xp[l1 * l1 + T.p[p].m1[z]] * gvp[l3 * l3 + T.p[p].m3[z]];
      if (T.p[p].m2[z] == l2 + 1) ax += cf * pr;
      else if (T.p[p].m2[z] == l2 - 1) ay += cf * pr;
    }
    gx += w[p] * ax;
    gy += w[p] * ay;
  }
}

// gx'^{l1}[m1] += w_p sum_{m3} CG_p[m1, 0, m3] (+-)Y_{l2}(z-hat) gv'^{l3}[m3]; with
// FLIP the edge direction is -z-hat in the frame (Y_l(-r) = (-1)^l Y_l(r))
template <int L, bool FLIP>
__host__ __device__ __forceinline__ void tpz_grad_x(const float* gvp, const float* w, float* gxp) {
  constexpr const cgc::Table& T = cgc::TableOf<L>::t;
#pragma unroll
  for (int p = 0; p < T.npaths; ++p) {
    const int l1 = T.p[p].l1, l2 = T.p[p].l2, l3 = T.p[p].l3;
    const double sg = (FLIP && (l2 & 1)) ? -1.0 : 1.0;
    float G[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int z = 0; z < T.p[p].nnz; ++z)
      if (T.p[p].m2[z] == l2)
        G[T.p[p].m1[z]] += (float)(T.p[p].v[z] * ypole(l2) * sg) * gvp[l3 * l3 + T.p[p].m3[z]];
#pragma unroll
    for (int m = 0; m < 2 * l1 + 1; ++m)
      if (pole_touch<L>(p, l2, m, true)) gxp[l1 * l1 + m] += w[p] * G[m];
  }
}

// ---------------------------------------------------------------- cross-lane sums
// Sums over aligned groups of W lanes, every lane of the group receiving the
// sum: DPP butterflies inside 16-lane rows, then the gfx950 permlane swaps
// across rows (v_permlane16_swap pairs rows 0-1 and 2-3, v_permlane32_swap the
// two wave halves).  No LDS traffic.  The row permutations are written as DPP
// updates with old value 0 and bound_ctrl set (every lane has a source in its
// row, so neither takes effect), the form the compiler folds into the consuming
// add as one v_add_f32_dpp.
__device__ __forceinline__ float dpp_add(float v, int ctrl_sel) {
  int b = __float_as_int(v);
  int r;
  switch (ctrl_sel) {
    case 0: r = __builtin_amdgcn_update_dpp(0, b, 0xB1, 0xF, 0xF, true); break;   // quad_perm [1,0,3,2]
    case 1: r = __builtin_amdgcn_update_dpp(0, b, 0x4E, 0xF, 0xF, true); break;   // quad_perm [2,3,0,1]
    case 2: r = __builtin_amdgcn_update_dpp(0, b, 0x141, 0xF, 0xF, true); break;  // row_half_mirror
    default: r = __builtin_amdgcn_update_dpp(0, b, 0x140, 0xF, 0xF, true); break; // row_mirror
  }
  return v + __int_as_float(r);
}

template <int W>
__device__ __forceinline__ float gsum(float v) {
  static_assert(W == 1 || W == 2 || W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "group width");
  if constexpr (W >= 2) v = dpp_add(v, 0);
  if constexpr (W >= 4) v = dpp_add(v, 1);
  if constexpr (W >= 8) v = dpp_add(v, 2);
  if constexpr (W >= 16) v = dpp_add(v, 3);
  if constexpr (W >= 32) {
    int b = __float_as_int(v);
    auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    v = __int_as_float(r[0]) + __int_as_float(r[1]);
  }
  if constexpr (W >= 64) {
    int b = __float_as_int(v);
    auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    v = __int_as_float(r[0]) + __int_as_float(r[1]);
  }
  return v;
}

// the partner's value from a permlane swap of s with itself: the pair holds s and the
// partner's s in an order fixed by the lane's row; either element equal to s works
__device__ __forceinline__ float swap_partner(float s, int r0, int r1) {
  return (r0 == __float_as_int(s)) ? __int_as_float(r1) : __int_as_float(r0);
}
__device__ __forceinline__ float dpp_get(float v, int ctrl_sel) {
  int b = __float_as_int(v);
  int r;
  switch (ctrl_sel) {
    case 0: r = __builtin_amdgcn_update_dpp(0, b, 0xB1, 0xF, 0xF, true); break;   // quad_perm [1,0,3,2]
    case 1: r = __builtin_amdgcn_update_dpp(0, b, 0x4E, 0xF, 0xF, true); break;   // quad_perm [2,3,0,1]
    case 2: r = __builtin_amdgcn_update_dpp(0, b, 0x141, 0xF, 0xF, true); break;  // row_half_mirror
    default: r = __builtin_amdgcn_update_dpp(0, b, 0x140, 0xF, 0xF, true); break; // row_mirror
  }
  return __int_as_float(r);
}

// Four sums over aligned groups of W lanes (16, 32 or 64) at once, reduce-scattered:
// afterwards every lane of quarter k of a group (lanes k W/4 .. (k+1) W/4 - 1) holds the
// group's sum of value k.  The first two exchanges halve the values carried (each lane
// sends what its partner keeps), the rest are plain butterflies: about half the work of
// four separate sums.
template <int W>
__device__ __forceinline__ float gsum4(float a, float b, float c, float d) {
  static_assert(W == 16 || W == 32 || W == 64, "group width");
  const int lane = (int)__lane_id();
  // one halving step: hi lanes keep (c, d) and send (a, b), lo lanes the reverse
  auto halve2 = [&](bool hi, float& x, float& y, auto exchange) {
    const float s1 = hi ? a : c, s2 = hi ? b : d;
    x = (hi ? c : a) + exchange(s1);
    y = (hi ? d : b) + exchange(s2);
  };
  auto halve1 = [&](bool hi, float x, float y, auto exchange) {
    const float s = hi ? x : y;
    return (hi ? y : x) + exchange(s);
  };
  auto perm32 = [](float s) {
    const int v = __float_as_int(s);
    auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return swap_partner(s, r[0], r[1]);
  };
  auto perm16 = [](float s) {
    const int v = __float_as_int(s);
    auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return swap_partner(s, r[0], r[1]);
  };
  float x, y, z;
  if constexpr (W == 64) {
    halve2((lane & 32) != 0, x, y, perm32);
    z = halve1((lane & 16) != 0, x, y, perm16);
    z += dpp_get(z, 3);
    z += dpp_get(z, 2);
    z += dpp_get(z, 1);
    z += dpp_get(z, 0);
  } else if constexpr (W == 32) {
    halve2((lane & 16) != 0, x, y, perm16);
    z = halve1((lane & 8) != 0, x, y, [](float s) { return dpp_get(s, 3); });
    z += dpp_get(z, 2);
    z += dpp_get(z, 1);
    z += dpp_get(z, 0);
  } else {
    halve2((lane & 8) != 0, x, y, [](float s) { return dpp_get(s, 3); });
    z = halve1((lane & 4) != 0, x, y, [](float s) { return dpp_get(s, 2); });
    z += dpp_get(z, 1);
    z += dpp_get(z, 0);
  }
  return z;
}

// runtime group width (a power of two <= 64; uniform across the wave)
__device__ __forceinline__ float gsum_rt(float v, int w) {
  switch (w) {
    case 1: return v;
    case 2: return gsum<2>(v);
    case 4: return gsum<4>(v);
    case 8: return gsum<8>(v);
    case 16: return gsum<16>(v);
    case 32: return gsum<32>(v);
    default: return gsum<64>(v);
  }
}

}  // namespace mdmp
