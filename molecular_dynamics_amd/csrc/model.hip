// Forward and backward kernels of the equivariant message-passing attention
// potential ("Ab Initio Accuracy Beyond the Cutoff", Abstract: equivariant
// message-passing Transformer layers, forces by back-propagation).
//
// Layout in HBM (all in sorted-slot order, atoms along the Hilbert curve):
//   features   [n][K][C]  (K = (lmax+1)^2, k = l^2 + m + l, channel fastest)
//   active edges (r < r_cut) compacted inside each row's padded range: row i's
//              active edges sit at row_ptr[i] .. aend[i] - 1, with a_j (sender),
//              a_r (padded index of the reverse edge), arev (reverse active
//              edge), geo [.][16]
//              float32 = r, u, du/dr, rhat[3], B[8], 0, 0
// Edge kernels run one block per (receiver row, channel block of 32 or 64
// channels), in an XCD-aware order.  Within a block, tiles of 16 or 32 edges go
// through
//   radial MLP: hidden SiLU(W_1 B) and W_2 on MFMA (16x16x4 fp32 or 16x16x32
//               bf16), staged through LDS as w'[e][p][c];
//   tensor product on VALU with lanes = channels, one edge per wave slot at
//               a time, Clebsch-Gordan nonzeros unrolled at compile time; the
//               unpruned layers take it in each edge's own frame (kernels.hpp);
//   online neighbour softmax per head (DPP / permlane sums) and segment sum kept
//   in registers; per-wave partial states merged through LDS at the row's end.
// Only the radial MLP is a dense contraction on the edge path ("Unlocking
// Tensor Core Performance", section "Batching and Tensor Shape Alignment":
// irregular sparse structure stays out of the matrix units); everything
// per edge stays on chip ("Kernel Fusion to Reduce Memory Pressure").
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "kernels.hpp"
#include "model.hpp"
#include "prof.hpp"

namespace mdmp {

static_assert(kGeoH == kGeoFloats, "geometry record size shared with the host");

// ====================================================================== geometry
// One 64-lane wave per row (4 rows per 256-thread block): lanes walk the row's padded
// edges 64 at a time, so index reads and writes are coalesced, and the active edges of
// a chunk are compacted with a ballot.
constexpr int kRowsPerBlock = 4;

__device__ __forceinline__ float wave_sum(float v) { return gsum<64>(v); }

// The calling wave's index in its (one-dimensional, whole-wave) block as a scalar: the
// compiler cannot prove threadIdx.x / 64 uniform, and with a scalar wave index the row
// indices, loop counters and weight addresses derived from it stay in scalar registers.
// The unpruned edge kernels keep the vector form (measured: their register allocation
// then ran slower, about 1.5 % in the forward and sender passes).
__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// the block's first row, in the XCD-aware order (chunks of 256 rows per XCD)
__device__ __forceinline__ int row_block0() {
  return (int)xcd_order(blockIdx.x, gridDim.x, 256 / kRowsPerBlock) * kRowsPerBlock;
}

// Active edges (r < r_cut) are compacted in order at the front of their row's padded
// range, so no count pass or scan is needed: the row's active range ends at aend[s].
// The 16-float geometry records of a chunk's active edges are staged in LDS and
// written out as consecutive 16-byte words.
__global__ __launch_bounds__(256) void k_active_fill(const float* __restrict__ pos, const int32_t* __restrict__ row_ptr,
                                                     const int32_t* __restrict__ col, const int32_t* __restrict__ rev,
                                                     int n, float Lbox, float rc, int32_t* __restrict__ aend,
                                                     int32_t* __restrict__ a_j, int32_t* __restrict__ a_r,
                                                     int32_t* __restrict__ amap, float* __restrict__ geo) {
  static_assert(kGeoH % 4 == 0, "records move as 16-byte words");
  __shared__ __align__(16) float s_rec[kRowsPerBlock][64 * kGeoH];
  const int w = wave_index(), lane = threadIdx.x & 63;
  const int s = row_block0() + w;
  if (s >= n) return;  // whole waves only: no block-wide barrier below
  const float inv_L = Lbox > 0.f ? 1.0f / Lbox : 0.f;  // L = 0: open boundary, no image shift
  const float norm = sqrtf(2.0f / rc);
  const float kpi = 3.14159265358979323846f / rc;
  float* rec = s_rec[w];
  int a0 = row_ptr[s];
  const int e1 = row_ptr[s + 1];
  const float sx = pos[3 * s], sy = pos[3 * s + 1], sz = pos[3 * s + 2];
  // one 64-edge chunk: activity test, ballot compaction, records staged in LDS and
  // copied out as 16-byte words
  auto chunk = [&](int e, int j, int re, float px, float py, float pz) {
    float dx, dy, dz, r = 0.f;
    bool act = false;
    if (e < e1) {
      min_image(px - sx, py - sy, pz - sz, Lbox, inv_L, dx, dy, dz);
      r = edge_r(dx, dy, dz);
      act = r < rc;
    }
    const uint64_t m = __ballot(act);
    if (m == 0) {
      if (e < e1) amap[e] = -1;
      return;
    }
    const int p = __popcll(m & ((1ull << (threadIdx.x & 63)) - 1ull));
    const int na = __popcll(m);
    if (e < e1) amap[e] = act ? a0 + p : -1;
    if (act) {
      a_j[a0 + p] = j;
      a_r[a0 + p] = re;
      float* g = rec + p * kGeoH;
      const float ir = 1.0f / r;
      const float x = dx * ir, y = dy * ir, z = dz * ir;
      const float d = r / rc, om = 1.0f - d;
      const float d2 = d * d, d5 = d2 * d2 * d;
      g[G_R] = r;
      g[G_U] = om * om * om * (1.0f + 3.0f * d + 6.0f * d2 + 10.0f * d2 * d + 15.0f * d2 * d2 + 21.0f * d5);
      g[G_DU] = -168.0f * d5 * om * om / rc;
      g[G_RH + 0] = x;
      g[G_RH + 1] = y;
      g[G_RH + 2] = z;
      {
        // sin(n t) for n = 1..8 from one sine/cosine pair: sin((n+1) t) = 2 cos t sin(n t) - sin((n-1) t)
        float s1, c1;
        sincosf(kpi * r, &s1, &c1);
        float sp = 0.f, sn = s1;
        const float nr = norm * ir;
#pragma unroll
        for (int q = 0; q < kNB; ++q) {
          g[G_B + q] = nr * sn;
          const float t = 2.0f * c1 * sn - sp;
          sp = sn;
          sn = t;
        }
      }
#pragma unroll
      for (int k = G_B + kNB; k < kGeoH; ++k) g[k] = 0.f;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const f4v* src = (const f4v*)rec;
    f4v* dst = (f4v*)(geo + (size_t)a0 * kGeoH);
    for (int t = threadIdx.x & 63; t < na * (kGeoH / 4); t += 64) dst[t] = src[t];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    a0 += na;
  };
  // two chunks per pass: both chunks' indices, then both chunks' sender positions, are
  // in flight before the first is processed
  for (int e0 = row_ptr[s]; e0 < e1; e0 += 128) {
    const int ea = e0 + lane, eb = e0 + 64 + lane;
    const int ja = ea < e1 ? col[ea] : s, jb = eb < e1 ? col[eb] : s;
    const int ra = ea < e1 ? rev[ea] : 0, rb = eb < e1 ? rev[eb] : 0;
    const float ax = pos[3 * ja], ay = pos[3 * ja + 1], az = pos[3 * ja + 2];
    const float bx = pos[3 * jb], by = pos[3 * jb + 1], bz = pos[3 * jb + 2];
    chunk(ea, ja, ra, ax, ay, az);
    if (e0 + 64 < e1) chunk(eb, jb, rb, bx, by, bz);
  }
  if ((threadIdx.x & 63) == 0) aend[s] = a0;
}

// arev[a]: the active slot of the reverse of active edge a (amap of its padded index)
__global__ __launch_bounds__(256) void k_arev(const int32_t* __restrict__ a_r, const int32_t* __restrict__ amap,
                                              const int32_t* __restrict__ abeg, const int32_t* __restrict__ aend,
                                              int n, int32_t* __restrict__ arev) {
  const int s = row_block0() + wave_index(), lane = threadIdx.x & 63;
  if (s >= n) return;
  for (int a = abeg[s] + lane; a < aend[s]; a += 64) arev[a] = amap[a_r[a]];
}

// ====================================================================== per-atom linears
// readout: one block of C threads handles kAPB atoms; its matrix is read transposed [in][out]
constexpr int kAPB = 8;

// h^0 = embedding row of the species, h^{l>0} = 0: one thread per (atom, 8 channels),
// each feature row written as 16-byte words.  Without ZERO_ROWS only h^0 is written (for a
// first layer that reads no other input row).
template <int K, int C, class TF, bool ZERO_ROWS = true>
__global__ __launch_bounds__(256) void k_embed(const float* __restrict__ emb, const int32_t* __restrict__ sp, int n,
                                               TF* __restrict__ h) {
  constexpr int V = 8, NV = C / V;
  static_assert(C % V == 0, "8-channel groups");
  const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= (int64_t)n * NV) return;
  const int i = (int)(x / NV), c0 = (int)(x % NV) * V;
  const float* e = emb + (size_t)sp[i] * C + c0;
  const f4v e0 = *(const f4v*)e, e1 = *(const f4v*)(e + 4);
  TF* o = h + (size_t)i * K * C + c0;
  if constexpr (sizeof(TF) == 2) {
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
    *(u4v*)o = u4v{pk2bf(e0.x, e0.y), pk2bf(e0.z, e0.w), pk2bf(e1.x, e1.y), pk2bf(e1.z, e1.w)};
#pragma unroll
    for (int k = 1; k < (ZERO_ROWS ? K : 1); ++k) *(u4v*)(o + k * C) = u4v{0u, 0u, 0u, 0u};
  } else {
    *(f4v*)o = e0;
    *(f4v*)(o + 4) = e1;
#pragma unroll
    for (int k = 1; k < (ZERO_ROWS ? K : 1); ++k) {
      *(f4v*)(o + k * C) = f4v{0.f, 0.f, 0.f, 0.f};
      *(f4v*)(o + k * C + 4) = f4v{0.f, 0.f, 0.f, 0.f};
    }
  }
}

// ------------------------------------------------------------------ per-atom products on MFMA
// Every per-atom product is y[a][o] = sum_i A[o][i] x[a][i] over a block of 16 atoms.  One
// MFMA tile computes D[o][a] for 16 output channels and the 16 atoms: the A operand holds
// rows of the weight matrix (global memory, row o0 + l % 16 in lane l), the B operand the
// atoms' input rows (staged in LDS, atom l % 16), and lane l receives D[4(l/16) + r][l % 16],
// i.e. channels o0 + 4(l/16) + r of atom l % 16.  Within a K-chunk, lane group g = l / 16
// reads one contiguous run of input channels (8 bf16 or 4 floats) from both operands: a
// permutation of the reduction index shared by A and B.  bf16 features use the 16x16x32
// bf16 MFMA (weights rounded to bf16 once, at model creation); float32 features use the
// 16x16x4 f32 MFMA.
constexpr int kNAT = 16;  // atoms per block
// waves per block: one 16-channel output tile per wave (at least 4 waves)
template <int C>
constexpr int atom_waves() {
  return C / 16 > 4 ? C / 16 : 4;
}

template <bool BF>
struct MM;
template <>
struct MM<true> {
  using F = s8v;
  using S = uint16_t;
  static constexpr int CK = 32, PAD = 8, EV = 8;
  static __device__ __forceinline__ F ld(const S* p, int g) { return *(const s8v*)(p + 8 * g); }
  static __device__ __forceinline__ f4v mma(f4v acc, F a, F b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, a), __builtin_bit_cast(bf8v, b), acc,
                                                   0, 0, 0);
  }
};
template <>
struct MM<false> {
  using F = f4v;
  using S = float;
  static constexpr int CK = 16, PAD = 4, EV = 4;
  static __device__ __forceinline__ F ld(const S* p, int g) { return *(const f4v*)(p + 4 * g); }
  static __device__ __forceinline__ f4v mma(f4v acc, F a, F b) {
#pragma unroll
    for (int z = 0; z < 4; ++z) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[z], b[z], acc, 0, 0, 0);
    return acc;
  }
};

template <bool BF>
__device__ __forceinline__ const typename MM<BF>::S* wsel(const float* f, const uint16_t* b) {
  if constexpr (BF)
    return b;
  else
    return f;
}

// A fragments of the 16-row tile starting at row0 (a matrix of ld columns, columns col0 ..)
// from its fragment-ordered copy, [rows/16][ld/CK][64 lanes][EV]: lane l of the fragment
// of row tile rt, column chunk cc holds row 16 rt + l mod 16, columns CK cc + EV (l / 16)
// .. + EV - 1 (LayerW's per-atom matrices are stored so)
template <bool BF, int NCH>
__device__ __forceinline__ void load_a(typename MM<BF>::F (&a)[NCH], const typename MM<BF>::S* __restrict__ w,
                                       int ld, int row0, int col0, int lane) {
  constexpr int CK = MM<BF>::CK, EV = MM<BF>::EV;
  const typename MM<BF>::S* p = w + ((size_t)((row0 / 16) * (ld / CK) + col0 / CK) * 64 + lane) * EV;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) a[ch] = *(const typename MM<BF>::F*)(p + (size_t)ch * 64 * EV);
}

template <bool BF, int NCH>
__device__ __forceinline__ f4v tile(f4v acc, const typename MM<BF>::F (&a)[NCH], const typename MM<BF>::S* brow,
                                    int g) {
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) acc = MM<BF>::mma(acc, a[ch], MM<BF>::ld(brow + ch * MM<BF>::CK, g));
  return acc;
}

// s[a][k0 + k][0 .. C) = x[n0 + a][k][0 .. C) for k < NK (rows of SK per atom in x); zero
// rows for atoms at or past n.
// NT threads: every thread issues all of its global loads before its first LDS store,
// so the block's whole tile is in flight at once.
template <int C, int KS, bool BF, int NK, int NT, int SK = NK, class SRC>
__device__ __forceinline__ void stage(typename MM<BF>::S* s, int k0, const SRC* __restrict__ x, int n0, int n) {
  using S = typename MM<BF>::S;
  constexpr int RS = C + MM<BF>::PAD, EV = MM<BF>::EV, VPR = C / EV;
  constexpr int per_atom = NK * VPR, TOT = kNAT * per_atom, IT = (TOT + NT - 1) / NT;
  constexpr bool SAME = sizeof(SRC) == sizeof(S);  // else float rows staged as bf16
  f4v v[IT][SAME ? 1 : 2];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int t = (int)threadIdx.x + it * NT;
    const int a = t / per_atom, r = t - a * per_atom;
    const int k = r / VPR, c = (r - k * VPR) * EV;
    const bool ld = (TOT % NT == 0 || t < TOT) && n0 + a < n;
    const SRC* p = x + ((size_t)(n0 + a) * SK + k) * C + c;
#pragma unroll
    for (int h = 0; h < (SAME ? 1 : 2); ++h) v[it][h] = ld ? *(const f4v*)(p + 4 * h) : f4v{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int t = (int)threadIdx.x + it * NT;
    if (TOT % NT != 0 && t >= TOT) break;
    const int a = t / per_atom, r = t - a * per_atom;
    const int k = r / VPR, c = (r - k * VPR) * EV;
    S* d = s + (a * KS + k0 + k) * RS + c;
    if constexpr (SAME) {
      *(f4v*)d = v[it][0];
    } else {
      s8v o;
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        o[z] = (short)f2bf(v[it][0][z]);
        o[4 + z] = (short)f2bf(v[it][1][z]);
      }
      *(s8v*)d = o;
    }
  }
}

// four consecutive channels of one atom row
__device__ __forceinline__ void st4(float* p, f4v v) { *(f4v*)p = v; }
__device__ __forceinline__ void st4(uint16_t* p, f4v v) {
  uint2 u;
  u.x = pk2bf(v[0], v[1]);
  u.y = pk2bf(v[2], v[3]);
  *(uint2*)p = u;
}
__device__ __forceinline__ f4v ld4(const float* p) { return *(const f4v*)p; }
__device__ __forceinline__ f4v ld4(const uint16_t* p) {
  const uint2 u = *(const uint2*)p;
  return f4v{bf2f((uint16_t)(u.x & 0xffffu)), bf2f((uint16_t)(u.x >> 16)), bf2f((uint16_t)(u.y & 0xffffu)),
             bf2f((uint16_t)(u.y >> 16))};
}
// four channels kept in their stored form (fewer registers while a load is held)
template <class TF>
struct Raw4;
template <>
struct Raw4<float> {
  using T = f4v;
  static __device__ __forceinline__ T ld(const float* p) { return *(const f4v*)p; }
  static __device__ __forceinline__ f4v cvt(T v) { return v; }
};
template <>
struct Raw4<uint16_t> {
  using T = uint2;
  static __device__ __forceinline__ T ld(const uint16_t* p) { return *(const uint2*)p; }
  static __device__ __forceinline__ f4v cvt(T u) {
    return f4v{bf2f((uint16_t)(u.x & 0xffffu)), bf2f((uint16_t)(u.x >> 16)), bf2f((uint16_t)(u.y & 0xffffu)),
               bf2f((uint16_t)(u.y >> 16))};
  }
};

// ht^l = W_v^l h^l, q = W_q h^0.  BOT (the first layer of an energy evaluation): its input
// is the embedding, whose rows l > 0 are zero, and its edge pass reads ht^0 only, so only
// ht^0 and q are formed.
template <int L, int C, class TF, bool BOT = false>
__global__ __launch_bounds__(atom_waves<C>() * 64) void k_pre_linear(const TF* __restrict__ h, int n, LayerW W, TF* __restrict__ ht,
                                                    float* __restrict__ q) {
  constexpr bool BF = std::is_same<TF, uint16_t>::value;
  using M = MM<BF>;
  using S = typename M::S;
  constexpr int K = Dims<L>::K, RS = C + M::PAD, NCH = C / M::CK;
  constexpr int LT = BOT ? 0 : L, KT = (LT + 1) * (LT + 1);  // rows read and formed per atom
  __shared__ __align__(16) S s_x[kNAT * KT * RS];
  const int n0 = blockIdx.x * kNAT;
  stage<C, KT, BF, KT, atom_waves<C>() * 64, K>(s_x, 0, h, n0, n);
  __syncthreads();
  const int wv = wave_index(), lane = threadIdx.x & 63, e = lane & 15, g = lane >> 4;
  const bool ok = n0 + e < n;
  const size_t row = (size_t)(n0 + e);
  const f4v zero = {0.f, 0.f, 0.f, 0.f};
  for (int ot = wv; ot < C / 16; ot += atom_waves<C>()) {
    const int o0 = 16 * ot, oc = o0 + 4 * g;
    typename M::F a[NCH];
#pragma unroll
    for (int l = 0; l <= LT; ++l) {
      load_a<BF>(a, wsel<BF>(W.wv[l], W.wv_b[l]), C, o0, 0, lane);
#pragma unroll
      for (int mm = 0; mm < 2 * l + 1; ++mm) {
        const int k = l * l + mm;
        const f4v d = tile<BF>(zero, a, s_x + (e * KT + k) * RS, g);
        if (ok) st4(ht + (row * K + k) * C + oc, d);
      }
    }
    load_a<BF>(a, wsel<BF>(W.wq, W.wq_b), C, o0, 0, lane);
    const f4v d = tile<BF>(zero, a, s_x + e * KT * RS, g);
    if (ok) st4(q + row * C + oc, d);
  }
}

// g_h^l += W_v^l^T g_ht^l ; g_h^0 += W_q^T g_q.  TOP (the last layer): the rows l > 0 of
// g_h hold no gradient yet (the readout reaches h^0 only, and its backward writes row 0
// alone), so they are written rather than accumulated.
template <int L, int C, class TF, bool TOP = false>
__global__ __launch_bounds__(atom_waves<C>() * 64) void k_pre_linear_bwd(const float* __restrict__ g_ht, const float* __restrict__ g_q,
                                                        int n, LayerW W, float* __restrict__ g_h) {
  constexpr bool BF = std::is_same<TF, uint16_t>::value;
  using M = MM<BF>;
  using S = typename M::S;
  constexpr int K = Dims<L>::K, KS = K + 1, RS = C + M::PAD, NCH = C / M::CK;
  __shared__ __align__(16) S s_x[kNAT * KS * RS];
  const int n0 = blockIdx.x * kNAT;
  stage<C, KS, BF, K, atom_waves<C>() * 64>(s_x, 0, g_ht, n0, n);
  stage<C, KS, BF, 1, atom_waves<C>() * 64>(s_x, K, g_q, n0, n);
  __syncthreads();
  const int wv = wave_index(), lane = threadIdx.x & 63, e = lane & 15, g = lane >> 4;
  const bool ok = n0 + e < n;
  const size_t row = (size_t)(n0 + e);
  const f4v zero = {0.f, 0.f, 0.f, 0.f};
  for (int ot = wv; ot < C / 16; ot += atom_waves<C>()) {
    const int i0 = 16 * ot, ic = i0 + 4 * g;
    typename M::F a[NCH];
#pragma unroll
    for (int l = 0; l <= L; ++l) {
      load_a<BF>(a, wsel<BF>(W.wvT[l], W.wvT_b[l]), C, i0, 0, lane);
#pragma unroll
      for (int mm = 0; mm < 2 * l + 1; ++mm) {
        const int k = l * l + mm;
        f4v d = tile<BF>(zero, a, s_x + (e * KS + k) * RS, g);
        if (k == 0) {
          typename M::F aq[NCH];
          load_a<BF>(aq, wsel<BF>(W.wqT, W.wqT_b), C, i0, 0, lane);
          d = tile<BF>(d, aq, s_x + (e * KS + K) * RS, g);
        }
        if (ok) {
          float* p = g_h + (row * K + k) * C + ic;
          st4(p, (TOP && l > 0) ? d : ld4(p) + d);
        }
      }
    }
  }
}

// h_out = h_in + update(m):  h^0 += SiLU(W_o^0 m^0);  h^l += sigmoid(W_g m^0)_l * W_o^l m^l.
// TOP (the last layer of an energy evaluation): only h^0 reaches the readout and the
// layer's messages have scalar rows only, so only the l = 0 rows are updated (the others
// would be left as they are: their update is W_o^l times a zero message).  BOT (the first
// layer): the input rows l > 0 are the embedding's zeros, so they are not read.
template <int L, int C, class TF, bool TOP = false, bool BOT = false>
__global__ __launch_bounds__(atom_waves<C>() * 64) void k_node_update(const TF* __restrict__ m, const TF* __restrict__ h_in, int n,
                                                     LayerW W, TF* __restrict__ h_out) {
  constexpr bool BF = std::is_same<TF, uint16_t>::value;
  using M = MM<BF>;
  using S = typename M::S;
  constexpr int K = Dims<L>::K, RS = C + M::PAD, NCH = C / M::CK;
  constexpr int LT = TOP ? 0 : L, KT = (LT + 1) * (LT + 1);  // rows updated per atom
  static_assert(C / 16 <= atom_waves<C>(), "one 16-channel output tile per wave");
  __shared__ __align__(16) S s_x[kNAT * KT * RS];
  const int n0 = blockIdx.x * kNAT;
  const int wv = wave_index(), lane = threadIdx.x & 63, e = lane & 15, g = lane >> 4;
  const bool ok = n0 + e < n, act = wv < C / 16;
  const size_t row = (size_t)(n0 + e);
  const int o0 = 16 * wv, oc = o0 + 4 * g;
  // the residual rows this lane updates, loaded before the staging so that both
  // streams are in flight together
  typename Raw4<TF>::T hr[KT];
#pragma unroll
  for (int k = 0; k < KT; ++k) hr[k] = typename Raw4<TF>::T{};
  if (act && ok) {
#pragma unroll
    for (int k = 0; k < (BOT ? 1 : KT); ++k) hr[k] = Raw4<TF>::ld(h_in + (row * K + k) * C + oc);
  }
  stage<C, KT, BF, KT, atom_waves<C>() * 64, K>(s_x, 0, m, n0, n);
  __syncthreads();
  if (!act) return;
  const f4v zero = {0.f, 0.f, 0.f, 0.f};
  typename M::F a[NCH];
  f4v gp[LT + 1];
#pragma unroll
  for (int l = 1; l <= LT; ++l) {
    load_a<BF>(a, wsel<BF>(W.wg, W.wg_b), C, (l - 1) * C + o0, 0, lane);
    gp[l] = tile<BF>(zero, a, s_x + e * KT * RS, g);
#pragma unroll
    for (int r = 0; r < 4; ++r) gp[l][r] = sigm(gp[l][r]);
  }
#pragma unroll
  for (int l = 0; l <= LT; ++l) {
    load_a<BF>(a, wsel<BF>(W.wo[l], W.wo_b[l]), C, o0, 0, lane);
#pragma unroll
    for (int mm = 0; mm < 2 * l + 1; ++mm) {
      const int k = l * l + mm;
      const f4v z = tile<BF>(zero, a, s_x + (e * KT + k) * RS, g);
      if (ok) {
        f4v v = Raw4<TF>::cvt(hr[k]);
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] += l == 0 ? silu(z[r]) : gp[l][r] * z[r];
        st4(h_out + (row * K + k) * C + oc, v);
      }
    }
  }
}

// backward of k_node_update: g_m from g_h (g_h itself passes through the residual).
// Phase 1 recomputes z = W_o m and the gate pre-activations into registers; phase 2 forms
// the elementwise gradients (gz^0 = g_h^0 SiLU'(z^0), gz^l = sigmoid(gp_l) g_h^l,
// g_gp_l = sigmoid'(gp_l) sum_m g_h^l z^l) in LDS, over the staged m; phase 3 contracts
// them with the transposed weights.
template <int L, int C, class TF, bool TOP = false>
__global__ __launch_bounds__(atom_waves<C>() * 64) void k_node_bwd(const TF* __restrict__ m, const float* __restrict__ g_h, int n,
                                                  LayerW W, float* __restrict__ g_m) {
  constexpr bool BF = std::is_same<TF, uint16_t>::value;
  using M = MM<BF>;
  using S = typename M::S;
  constexpr int K = Dims<L>::K, RS = C + M::PAD, NCH = C / M::CK;
  // TOP (the last layer): g_h and the messages have scalar rows only, and only g_m^0 is read
  constexpr int LT = TOP ? 0 : L, KT = (LT + 1) * (LT + 1), KG = KT + LT;
  static_assert(C / 16 <= atom_waves<C>(), "one 16-channel output tile per wave");
  __shared__ __align__(16) S s[kNAT * KG * RS];
  const int n0 = blockIdx.x * kNAT;
  const int wv = wave_index(), lane = threadIdx.x & 63, e = lane & 15, g = lane >> 4;
  const bool ok = n0 + e < n, act = wv < C / 16;
  const size_t row = (size_t)(n0 + e);
  const f4v zero = {0.f, 0.f, 0.f, 0.f};
  const int o0 = 16 * wv, oc = o0 + 4 * g;
  // the incoming gradient rows of this lane, loaded before the staging so that both
  // streams are in flight together
  f4v gl[KT];
#pragma unroll
  for (int k = 0; k < KT; ++k) gl[k] = act && ok ? ld4(g_h + (row * K + k) * C + oc) : zero;
  stage<C, KG, BF, KT, atom_waves<C>() * 64, K>(s, 0, m, n0, n);
  __syncthreads();
  f4v z[KT], gp[LT + 1];
  if (act) {
    typename M::F a[NCH];
#pragma unroll
    for (int l = 1; l <= LT; ++l) {
      load_a<BF>(a, wsel<BF>(W.wg, W.wg_b), C, (l - 1) * C + o0, 0, lane);
      gp[l] = tile<BF>(zero, a, s + e * KG * RS, g);
    }
#pragma unroll
    for (int l = 0; l <= LT; ++l) {
      load_a<BF>(a, wsel<BF>(W.wo[l], W.wo_b[l]), C, o0, 0, lane);
#pragma unroll
      for (int mm = 0; mm < 2 * l + 1; ++mm) z[l * l + mm] = tile<BF>(zero, a, s + (e * KG + l * l + mm) * RS, g);
    }
  }
  __syncthreads();  // the staged m is overwritten below
  if (act) {
    S* srow = s + e * KG * RS + oc;
    {
      f4v v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = gl[0][r] * dsilu(z[0][r]);
      st4(srow, v);
    }
#pragma unroll
    for (int l = 1; l <= LT; ++l) {
      f4v sg, gg = zero;
#pragma unroll
      for (int r = 0; r < 4; ++r) sg[r] = sigm(gp[l][r]);
#pragma unroll
      for (int mm = 0; mm < 2 * l + 1; ++mm) {
        const int k = l * l + mm;
        f4v v;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = sg[r] * gl[k][r];
          gg[r] += gl[k][r] * z[k][r];
        }
        st4(srow + k * RS, v);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) gg[r] *= sg[r] * (1.0f - sg[r]);
      st4(srow + (KT + l - 1) * RS, gg);
    }
  }
  __syncthreads();
  // g_m^l[i] = sum_o W_o^l[o][i] gz^l[o];  g_m^0[i] += sum_l sum_o W_g^l[o][i] g_gp_l[o]
  for (int ot = wv; ot < C / 16; ot += atom_waves<C>()) {
    const int i0 = 16 * ot, ic = i0 + 4 * g;
    typename M::F a[NCH];
#pragma unroll
    for (int l = 0; l <= LT; ++l) {
      load_a<BF>(a, wsel<BF>(W.woT[l], W.woT_b[l]), C, i0, 0, lane);
#pragma unroll
      for (int mm = 0; mm < 2 * l + 1; ++mm) {
        const int k = l * l + mm;
        f4v d = tile<BF>(zero, a, s + (e * KG + k) * RS, g);
        if (k == 0) {
#pragma unroll
          for (int lg = 1; lg <= LT; ++lg) {
            typename M::F ag[NCH];
            load_a<BF>(ag, wsel<BF>(W.wgT, W.wgT_b), L * C, i0, (lg - 1) * C, lane);
            d = tile<BF>(d, ag, s + (e * KG + KT + lg - 1) * RS, g);
          }
        }
        if (ok) st4(g_m + (row * K + k) * C + ic, d);
      }
    }
  }
}

// E_i^k = sum_c w_out^k[c] SiLU((W_r^k h_i^0)[c]) for readout heads k = 0..R-1 on the
// same features ("Exascale Multi-Task Graph Foundation Models", Fig. 5: the encoder
// runs once, every head reads its output); head k's matrix at wrT + k C^2 ([in][out]),
// its output weights at wout + k C; e_atoms[k n + i].  R = 1 is the model's own readout.
template <int C, class TF>
__global__ __launch_bounds__(C) void k_readout(const TF* __restrict__ h, int n, int K, int R,
                                               const float* __restrict__ wrT, const float* __restrict__ wout,
                                               float* __restrict__ e_atoms) {
  __shared__ float s_x[kAPB][C];
  __shared__ float s_red[kAPB][C];
  const int c = threadIdx.x;
  const int n0 = blockIdx.x * kAPB;
  for (int a = 0; a < kAPB; ++a)
    s_x[a][c] = (n0 + a < n) ? FeatIO<TF>::ld(h + (size_t)(n0 + a) * K * C + c) : 0.f;
  __syncthreads();
  for (int k = 0; k < R; ++k) {
    const float* wk = wrT + (size_t)k * C * C;
    float z[kAPB];
#pragma unroll
    for (int a = 0; a < kAPB; ++a) z[a] = 0.f;
    for (int ci = 0; ci < C; ++ci) {
      const float w = wk[ci * C + c];
#pragma unroll
      for (int a = 0; a < kAPB; ++a) z[a] += w * s_x[a][ci];
    }
    const float wo = wout[k * C + c];
#pragma unroll
    for (int a = 0; a < kAPB; ++a) s_red[a][c] = wo * silu(z[a]);
    __syncthreads();
    if (c < kAPB && n0 + c < n) {
      float s = 0.f;
      for (int q = 0; q < C; ++q) s += s_red[c][q];
      e_atoms[(size_t)k * n + n0 + c] = s;
    }
    __syncthreads();
  }
}

// gradient of sum_k lam_k sum_i E_i^k with respect to h^0 (lam = nullptr: every
// lam_k = 1): sum_k lam_k W_r^kT (w_out^k * SiLU'(W_r^k h^0)); h^{l>0} get zero
template <int C, class TF>
__global__ __launch_bounds__(C) void k_readout_bwd(const TF* __restrict__ h, int n, int K, int R,
                                                   const float* __restrict__ wrT, const float* __restrict__ wr,
                                                   const float* __restrict__ wout, const float* __restrict__ lam,
                                                   float* __restrict__ g_h) {
  __shared__ float s_x[kAPB][C];
  __shared__ float s_g[kAPB][C];
  const int c = threadIdx.x;
  const int n0 = blockIdx.x * kAPB;
  for (int a = 0; a < kAPB; ++a)
    s_x[a][c] = (n0 + a < n) ? FeatIO<TF>::ld(h + (size_t)(n0 + a) * K * C + c) : 0.f;
  __syncthreads();
  float acc[kAPB];
#pragma unroll
  for (int a = 0; a < kAPB; ++a) acc[a] = 0.f;
  for (int k = 0; k < R; ++k) {
    const float* wk = wrT + (size_t)k * C * C;
    float z[kAPB];
#pragma unroll
    for (int a = 0; a < kAPB; ++a) z[a] = 0.f;
    for (int ci = 0; ci < C; ++ci) {
      const float w = wk[ci * C + c];
#pragma unroll
      for (int a = 0; a < kAPB; ++a) z[a] += w * s_x[a][ci];
    }
    const float wo = wout[k * C + c] * (lam ? lam[k] : 1.0f);
#pragma unroll
    for (int a = 0; a < kAPB; ++a) s_g[a][c] = wo * dsilu(z[a]);
    __syncthreads();
    const float* wrk = wr + (size_t)k * C * C;
    for (int co = 0; co < C; ++co) {
      const float w = wrk[co * C + c];
#pragma unroll
      for (int a = 0; a < kAPB; ++a) acc[a] += w * s_g[a][co];
    }
    __syncthreads();
  }
  // row 0 only: the rows l > 0 carry no gradient at the top, and the top layer's node
  // backward and pre-linear backward neither read nor accumulate into them
#pragma unroll
  for (int a = 0; a < kAPB; ++a) {
    if (n0 + a >= n) break;
    g_h[(size_t)(n0 + a) * K * C + c] = acc[a];
  }
}

// fixed-order float64 sum of per-atom energies (one block)
__global__ __launch_bounds__(1024) void k_energy_sum(const float* __restrict__ e_atoms, int n,
                                                     double* __restrict__ out) {
  __shared__ double sh[1024];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += 1024) s += (double)e_atoms[i];
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = sh[0];
}

// hidden units of a tile in LDS: float rows of kHR + 1, or bf16 rows of kHR + 8
// (16-byte aligned, read as MFMA operands directly)
template <class HT>
constexpr int hid_stride() {
  return sizeof(HT) == 2 ? kHR + 8 : kHR + 1;
}

// With ON, the weight pointer passes through an empty asm statement at each use, so
// the per-lane fragment addresses are formed inside the tile loop instead of being
// hoisted out of it and held (or spilled) across the whole row.  Used where the
// kernel would otherwise spill (float32 features, pruned layers); the unpruned bf16
// kernels keep the hoisted addresses.
template <bool ON, class T>
__device__ __forceinline__ const T* per_tile(const T* p) {
  if constexpr (ON) asm volatile("" : "+s"(p));
  return p;
}
template <int MODE, bool BF>
constexpr bool kPerTile = !BF || MODE != 0;
// The same for a pointer that must stay a global-memory pointer (its loads global, not
// flat loads, which would also count against the LDS wait counter).
template <class T>
__device__ __forceinline__ const T* per_tile_global(const T* p) {
  auto gp = (const __attribute__((address_space(1))) T*)p;
  asm volatile("" : "+s"(gp));
  return (const T*)gp;
}

// Sum over one attention head's channels (aligned groups of dh lanes): DHC > 0 fixes
// dh at compile time (straight-line DPP), DHC = 0 takes the runtime width.
template <int DHC>
__device__ __forceinline__ float head_sum(float v, int dh) {
  if constexpr (DHC > 0) return gsum<DHC>(v);
  else return gsum_rt(v, dh);
}

// ====================================================================== radial MLP on MFMA
// w'[e][q][c] = (W_2 s_e)[p(q)*C + cbase + c] for the edges of a tile and the
// active paths q, stored as WT (bf16 for bf16 features, else float).  A = W_2 rows
// (p, c), B = hidden s^T, D = w'^T: lane l holds D[4(l/16)+r][l%16].  The reduction
// index is permuted so each lane reads 16 consecutive hidden units (one 64-byte row
// segment of W_2).
//
// Edge stride (elements) of the w' tile in LDS: NA*CB padded so that the MFMA
// output stores (16 edges x 4 lane groups, w = 2 or 4 dwords each) spread evenly
// over the 64 banks: the stride in dwords, modulo 64, has gcd 4w with 64.
constexpr int cgcd(int a, int b) { return b == 0 ? a : cgcd(b, a % b); }
template <int NA, int CB, bool BF>
constexpr int sw_stride() {
  constexpr int esz = BF ? 2 : 4, w = BF ? 2 : 4;
  int dw = NA * CB * esz / 4;
  while (cgcd(dw % 64, 64) != 4 * w) dw += w;
  return dw * 4 / esz;
}
static_assert(sw_stride<15, 64, true>() == 976 && sw_stride<3, 64, true>() == 208, "w' strides");

// SWZ: w2b is the fragment-ordered copy (LayerW::w2sw) of an unpruned bf16 layer
template <int L, int MODE, int C, int CB, bool BF, int TE, bool SWZ = false, class HT>
__device__ __forceinline__ void radial_w(const float* __restrict__ w2, const uint16_t* __restrict__ w2b, int cbase,
                                         const HT* s_hid, std::conditional_t<BF, uint16_t, float>* s_w, int wv,
                                         int lane) {
  constexpr int HS = hid_stride<HT>();
  constexpr int NA = Paths<L, MODE>::count();
  constexpr int SWE = sw_stride<NA, CB, BF>();
  constexpr int NRB = NA * CB / 16;
  constexpr int NEB = TE / 16;  // 16-edge column blocks; each W_2 fragment is reused for all of them
  const int e = lane & 15, g = lane >> 4;
  if constexpr (!BF) {
    w2 = per_tile<kPerTile<MODE, BF>>(w2);
    const int lane_off = e * kHR + 16 * g;  // the lane's part of the fragment address
    auto* w_lane = s_w + e * SWE + 4 * g;   // and of the w' tile address
    for (int rb = wv; rb < NRB; rb += kNW) {
      const int q = (rb * 16) / CB, c0 = (rb * 16) % CB;
      const int p = path_of<L, MODE>(q);
      const f4v* Ar = SWZ ? (const f4v*)w2 + ((size_t)((cbase / CB) * NRB + rb) * 4) * 64 + lane
                          : MODE == 0 ? (const f4v*)(w2 + ((size_t)(p * C + cbase + c0 + e)) * kHR + 16 * g)
                                      : (const f4v*)(w2 + (size_t)(p * C + cbase + c0) * kHR + lane_off);
      constexpr int AS = SWZ ? 64 : 1;  // f4v stride of the lane's four loads
      f4v a0 = Ar[0], a1 = Ar[AS], a2 = Ar[2 * AS], a3 = Ar[3 * AS];
      float af[16] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3],
                      a2[0], a2[1], a2[2], a2[3], a3[0], a3[1], a3[2], a3[3]};
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb) {
        const int ee = 16 * eb + e;
        f4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 16; ++t)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af[t], FeatIO<HT>::ld(s_hid + ee * HS + 16 * g + t), acc, 0, 0,
                                                     0);
        if constexpr (MODE == 0)
          st4(s_w + ee * SWE + q * CB + c0 + 4 * g, acc);
        else
          st4(w_lane + 16 * eb * SWE + q * CB + c0, acc);
      }
    }
  } else {
    w2b = per_tile<kPerTile<MODE, BF>>(w2b);
    const int lane_off = e * kHR + 16 * g;  // the lane's part of the fragment address
    auto* w_lane = s_w + e * SWE + 4 * g;   // and of the w' tile address
    for (int rb = wv; rb < NRB; rb += kNW) {
      const int q = (rb * 16) / CB, c0 = (rb * 16) % CB;
      const int p = path_of<L, MODE>(q);
      const s8v* Ar = SWZ ? (const s8v*)w2b + ((size_t)((cbase / CB) * NRB + rb) * 2) * 64 + lane
                          : MODE == 0 ? (const s8v*)(w2b + ((size_t)(p * C + cbase + c0 + e)) * kHR + 16 * g)
                                      : (const s8v*)(w2b + (size_t)(p * C + cbase + c0) * kHR + lane_off);
      s8v a0 = Ar[0], a1 = Ar[SWZ ? 64 : 1];
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb) {
        const int ee = 16 * eb + e;
        s8v b0, b1;
        if constexpr (sizeof(HT) == 2) {
          b0 = *(const s8v*)(s_hid + ee * HS + 16 * g);
          b1 = *(const s8v*)(s_hid + ee * HS + 16 * g + 8);
        } else {
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            b0[t] = (short)f2bf(s_hid[ee * HS + 16 * g + t]);
            b1[t] = (short)f2bf(s_hid[ee * HS + 16 * g + 8 + t]);
          }
        }
        f4v acc = {0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, a0), __builtin_bit_cast(bf8v, b0), acc,
                                                      0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, a1), __builtin_bit_cast(bf8v, b1), acc,
                                                      0, 0, 0);
        if constexpr (MODE == 0)
          st4(s_w + ee * SWE + q * CB + c0 + 4 * g, acc);
        else
          st4(w_lane + 16 * eb * SWE + q * CB + c0, acc);
      }
    }
  }
}

// The first of a wave's bf16 W_2^T fragments for radial_w_bwd, requested before the
// barrier that precedes the product, so the product starts on fragments in hand while
// the rest stream in as before.  Three of them: all fifteen at once measured slower
// than none (every wave's requests then arrive together), six gained less than three.
template <int L, int MODE, int C, int CB, bool SWZ = false>
struct W2tFrags {
  static constexpr int NALL = Paths<L, MODE>::count() * CB / 32;
  static constexpr int NT = NALL < 3 ? NALL : 3;
  s8v a[NT];
  // SWZ: w2tb is the fragment-ordered copy (LayerW::w2tsw)
  __device__ __forceinline__ void fetch(const uint16_t* __restrict__ w2tb, int cbase, int wv, int lane) {
    constexpr int PC = cgc::TableOf<L>::t.npaths * C;
    const int g = lane >> 4, h = 16 * wv + (lane & 15);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int k = 32 * t + 8 * g;
      a[t] = SWZ ? ((const s8v*)w2tb)[((size_t)((cbase / CB) * 4 + wv) * NALL + t) * 64 + lane]
                 : *(const s8v*)(w2tb + (size_t)h * PC + path_of<L, MODE>(q_of(k)) * C + cbase + k % CB);
    }
  }
  static __device__ __forceinline__ int q_of(int k) { return k / CB; }
};

// g_s[e][h] = sum_{q,c} gw[e][q][c] W_2[p(q)*C + cbase + c][h], from the transposed
// copy W_2^T [64][P*C]: A = W_2^T rows (hidden units), B = gw^T, D = g_s^T.
// Wave wv owns hidden units 16 wv .. 16 wv + 15; acc[eb][r] is unit 16 wv + 4 (lane/16)
// + r of edge 16 eb + lane%16, the layout of radial_pre().
// SWZ: w2tb is the fragment-ordered copy (LayerW::w2tsw) of an unpruned bf16 layer
template <int L, int MODE, int C, int CB, bool BF, int TE, bool SWZ = false>
__device__ __forceinline__ void radial_w_bwd(const float* __restrict__ w2t, const uint16_t* __restrict__ w2tb,
                                             int cbase, const std::conditional_t<BF, uint16_t, float>* s_gw,
                                             f4v* acc /*[TE/16]*/, int wv, int lane, const s8v* frag = nullptr) {
  constexpr int NA = Paths<L, MODE>::count();
  constexpr int KT = NA * CB;
  constexpr int SWE = sw_stride<NA, CB, BF>();
  constexpr int PC = cgc::TableOf<L>::t.npaths * C;
  constexpr int NEB = TE / 16;
  const int e = lane & 15, g = lane >> 4;
  const int h = 16 * wv + (lane & 15);
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb) acc[eb] = f4v{0.f, 0.f, 0.f, 0.f};
  if constexpr (!BF) {
    // lane group g walks k = g*KT/4 .. (g+1)*KT/4 - 1, four at a time
    static_assert(KT % 16 == 0, "k range");
    w2t = per_tile<kPerTile<MODE, BF>>(w2t);
    const int k0 = g * (KT / 4);
#pragma unroll 2
    for (int t = 0; t < KT / 4; t += 4) {
      const int k = k0 + t;
      const int q = k / CB, c = k % CB;
      const f4v a = SWZ ? ((const f4v*)w2t)[((size_t)((cbase / CB) * 4 + wv) * (KT / 16) + t / 4) * 64 + lane]
                        : *(const f4v*)(w2t + (size_t)h * PC + path_of<L, MODE>(q) * C + cbase + c);
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb) {
        const f4v b = *(const f4v*)(s_gw + (16 * eb + e) * SWE + k);
#pragma unroll
        for (int z = 0; z < 4; ++z) acc[eb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[z], b[z], acc[eb], 0, 0, 0);
      }
    }
  } else {
    static_assert(KT % 32 == 0, "k range");
    // the fragment-ordered copy's loads would be hoisted out of the tile loop as a whole
    // (registers for all of them): its base is made opaque per tile
    if constexpr (SWZ) w2tb = per_tile_global(w2tb);
    else w2tb = per_tile<kPerTile<MODE, BF>>(w2tb);
    for (int t = 0; t < KT / 32; ++t) {
      const int k = 32 * t + 8 * g;
      const int q = k / CB, c = k % CB;
      const s8v a = (frag && t < W2tFrags<L, MODE, C, CB>::NT) ? frag[t < W2tFrags<L, MODE, C, CB>::NT ? t : 0]
                    : SWZ ? ((const s8v*)w2tb)[((size_t)((cbase / CB) * 4 + wv) * (KT / 32) + t) * 64 + lane]
                          : *(const s8v*)(w2tb + (size_t)h * PC + path_of<L, MODE>(q) * C + cbase + c);
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb) {
        const s8v b = *(const s8v*)(s_gw + (16 * eb + e) * SWE + k);
        acc[eb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8v, a), __builtin_bit_cast(bf8v, b),
                                                          acc[eb], 0, 0, 0);
      }
    }
  }
}

// Pre-activations of the radial MLP's hidden layer for the tile, W_1 B^T on the
// 16x16x4 float32 MFMA (K = the 8 Bessel values): wave wv owns hidden units
// 16 wv .. 16 wv + 15 and pre[eb][r] is unit 16 wv + 4 (lane/16) + r of edge
// 16 eb + lane%16 (A = W_1 rows, B = Bessel values of the tile's edges).
template <int TE, bool PT>
__device__ __forceinline__ void radial_pre(const float* __restrict__ w1, const float* s_geo, int wv, int lane,
                                           f4v* pre /*[TE/16]*/) {
  static_assert(kHR == 16 * kNW && kNB == 8, "one 16-unit block per wave, K = 8");
  const int m = lane & 15, g = lane >> 4;
  w1 = per_tile<PT>(w1);
  const float a0 = w1[(16 * wv + m) * kNB + g], a1 = w1[(16 * wv + m) * kNB + 4 + g];
#pragma unroll
  for (int eb = 0; eb < TE / 16; ++eb) {
    const float* b = s_geo + (16 * eb + m) * kGeo + G_B;
    f4v acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b[g], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b[4 + g], acc, 0, 0, 0);
    pre[eb] = acc;
  }
}

// the hidden layer of the radial MLP for a tile whose geometry is in LDS
template <int TE, bool PT, bool SW = false, class HT>
__device__ __forceinline__ void tile_hidden(const float* __restrict__ w1, const float* s_geo, HT* s_hid, int tid) {
  const int wv = SW ? wave_index() : tid >> 6, lane = tid & 63;
  f4v pre[TE / 16];
  radial_pre<TE, PT>(w1, s_geo, wv, lane, pre);
#pragma unroll
  for (int eb = 0; eb < TE / 16; ++eb) {
    HT* o = s_hid + (16 * eb + (lane & 15)) * hid_stride<HT>() + 16 * wv + 4 * (lane >> 4);
    if constexpr (sizeof(HT) == 2) {
      // four consecutive units: one 8-byte store (row stride and offset are multiples of 8 bytes)
      const uint32_t lo = pk2bf(silu(pre[eb][0]), silu(pre[eb][1]));
      const uint32_t hi = pk2bf(silu(pre[eb][2]), silu(pre[eb][3]));
      *(uint2*)o = make_uint2(lo, hi);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = silu(pre[eb][r]);
    }
  }
  __syncthreads();
}

// load a tile's geometry and the hidden layer of the radial MLP; YL >= 0: also the
// harmonics Y (l <= YL) of each edge direction into the record's G_Y slots (lab-frame
// layers; the edge-frame layers put their rotation there instead)
template <int TE, bool PT, int YL, class HT>
__device__ __forceinline__ void load_tile(const float* __restrict__ geo, const int32_t* __restrict__ a_j,
                                          const int32_t* __restrict__ extra, int t0, int nv, int self,
                                          const float* __restrict__ w1, float* s_geo, int* s_j, int* s_x,
                                          HT* s_hid, int tid) {
  // 16-edge tiles: one 16-byte word of a record per thread, from a base that passes an
  // empty asm statement (the per-lane address is rebuilt per tile, not hoisted out of
  // the tile loop); 32-edge tiles: a loop over the LDS rows (kGeo floats) that skips the
  // slots the HBM record lacks.  Either choice the other way round spills in the
  // unpruned receiver pass.
  if constexpr (TE == 16) {
    geo = per_tile<true>(geo);
    if (tid < TE * (kGeoH / 4)) {
      const int e = tid / (kGeoH / 4), f = 4 * (tid % (kGeoH / 4));
      const f4v v = e < nv ? *(const f4v*)(geo + (size_t)(t0 + e) * kGeoH + f) : f4v{0.f, 0.f, 0.f, 0.f};
      *(f4v*)(s_geo + e * kGeo + f) = v;
    }
  } else {
    for (int x = tid; x < TE * kGeo; x += 256) {
      const int e = x / kGeo, f = x % kGeo;
      if (f < kGeoH) s_geo[x] = e < nv ? geo[(size_t)(t0 + e) * kGeoH + f] : 0.f;
    }
  }
  if (tid < TE) {
    s_j[tid] = tid < nv ? a_j[t0 + tid] : self;
    if (extra) s_x[tid] = tid < nv ? extra[t0 + tid] : 0;
  }
  __syncthreads();
  if constexpr (YL >= 0) {
    if (tid < nv) {
      float* g = s_geo + tid * kGeo;
      float Y[Dims<YL>::K];
      real_sh<YL>(g[G_RH], g[G_RH + 1], g[G_RH + 2], Y);
#pragma unroll
      for (int k = 0; k < Dims<YL>::K; ++k) g[G_Y + k] = Y[k];
    }
  }
  tile_hidden<TE, PT, (YL >= 0)>(w1, s_geo, s_hid, tid);  // ends with a block barrier
}

// A tile's geometry records and sender indices gathered into registers one tile ahead
// (issued before the current tile's edge loop, stored to LDS at the next tile).
template <int TE, bool EXTRA = false>
struct TileAhead {
  // one 8-byte pair of a record per thread
  static constexpr int NP = TE * kGeoH / 2;
  static_assert(NP <= 256, "a tile's records in one pass");
  float2 g = make_float2(0.f, 0.f);
  int j = 0, x = 0;
  __device__ __forceinline__ void fetch(const float* __restrict__ geo, const int32_t* __restrict__ a_j,
                                        const int32_t* __restrict__ extra, int t0, int nv, int self, int tid) {
    // with EXTRA (the sender pass) an opaque base per call: the per-lane record addresses
    // are rebuilt from it here instead of being hoisted out of the tile loop as 64-bit
    // values, which spill in that register-bound kernel
    geo = per_tile<EXTRA>(geo);
    if (tid < NP) {
      const int e = tid / (kGeoH / 2);
      g = e < nv ? *(const float2*)(geo + (size_t)(t0 + e) * kGeoH + 2 * (tid % (kGeoH / 2))) : make_float2(0.f, 0.f);
    }
    if (tid < TE) {
      j = tid < nv ? a_j[t0 + tid] : self;
      if constexpr (EXTRA) x = tid < nv ? extra[t0 + tid] : 0;
    }
  }
  __device__ __forceinline__ void store(float* s_geo, int* s_j, int* s_x, int tid) const {
    if (tid < NP) *(float2*)(s_geo + (tid / (kGeoH / 2)) * kGeo + 2 * (tid % (kGeoH / 2))) = g;
    if (tid < TE) {
      s_j[tid] = j;
      if constexpr (EXTRA) s_x[tid] = x;
    }
  }
};

// Forward and sender passes: 32-edge tiles (16 for the float32 unpruned layers,
// whose w' tile would not fit), so each W_2 fragment loaded from L2 serves two
// 16-edge column blocks; 32-channel blocks for the unpruned layers (the w' tile of
// 32 edges x 15 paths in 31 KB) and for float32, 64 for the pruned bf16 layers.
// The receiver pass uses the same tiles (edge_channel_block() is the narrowest
// channel block of any pass).
template <int MODE, bool BF>
constexpr int fs_channel_block(int C) {
  return (BF && MODE != 0) ? (C < 64 ? C : 64) : (C < 32 ? C : 32);
}
// Whether the first layer's receiver pass (MODE & 1) folds each odd 32-channel slot of
// the geometry-gradient partials into the even one: its channel blocks span two slots.
template <int MODE, bool BF>
constexpr bool fold_slot_pairs(int C) {
  return (MODE & 1) != 0 && fs_channel_block<MODE, BF>(C) == 2 * edge_channel_block(C, BF);
}
template <int MODE, bool BF>
constexpr int fs_tile_edges() {
  return (BF || MODE != 0) ? 2 * kTE : kTE;
}

// ====================================================================== edge forward
template <int L, int MODE, int C, class TF, int DHC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MODE == 0 ? 4 : (sizeof(TF) == 2 ? 7 : 6)))) void k_edge_fwd(EdgeArgs A, LayerW W, TF* __restrict__ m_out) {
  constexpr int TE = fs_tile_edges<MODE, sizeof(TF) == 2>();
  constexpr int K = Dims<L>::K, NA = Paths<L, MODE>::count();
  constexpr int KX = (MODE & 1) ? 1 : K;  // inputs that can be nonzero
  constexpr int KV = (MODE & 2) ? 1 : K;  // outputs that are needed
  constexpr int CB = fs_channel_block<MODE, sizeof(TF) == 2>(C);
  constexpr int EPW = 64 / CB, NS = kNW * EPW;
  constexpr bool BF = sizeof(TF) == 2;
  constexpr bool SWZ = MODE <= 2 && C >= 32;  // fragment-ordered W_2 copies
  __shared__ __align__(16) float s_geo[TE * kGeo];
  __shared__ int s_j[TE];
  using HT = std::conditional_t<BF, uint16_t, float>;  // hidden units stored as the MFMA reads them
  __shared__ __align__(16) HT s_hid[TE * hid_stride<HT>()];
  using WT = std::conditional_t<BF, uint16_t, float>;  // w' of the tile; the same storage merges the slots
  constexpr int SWE = sw_stride<NA, CB, BF>();
  constexpr int SWB = std::max<int>(TE * SWE * sizeof(WT), 256 * (KV + 2) * sizeof(float));
  __shared__ __align__(16) unsigned char s_wb[SWB];
  WT* s_w = (WT*)s_wb;
  int i, cblk;
  xcd_row_block(i, cblk);
  const int cbase = cblk * CB;
  const int tid = threadIdx.x, wv = MODE == 0 ? tid >> 6 : wave_index(), lane = tid & 63;
  const int slot = lane / CB, c = lane % CB, sl = wv * EPW + slot;
  const int DH = DHC > 0 ? DHC : A.dh;
  const float rs = rsqrtf((float)DH);
  const float qc = A.q[(size_t)i * C + cbase + c];
  const TF* __restrict__ ht = (const TF*)A.ht;
  const int a0 = A.abeg[i], a1 = A.aend[i];
  constexpr bool EF = MODE == 0;  // unpruned layers: products in each edge's own frame
  float* s_d2 = (float*)s_hid;    // l = 2 rotation blocks, once the hidden tile is consumed
  static_assert(TE * kD2 * sizeof(float) <= sizeof(s_hid), "rotation blocks fit");
  float Mx = -INFINITY, Zs = 0.f, macc[KV];
#pragma unroll
  for (int k = 0; k < KV; ++k) macc[k] = 0.f;
  // unpruned layers gather the next tile's geometry during the current tile
  constexpr bool TA = MODE == 0;
  TileAhead<TE> ahead;
  if (TA && a0 < a1) ahead.fetch(A.geo, A.a_j, nullptr, a0, min(TE, a1 - a0), i, tid);
  for (int t0 = a0; t0 < a1; t0 += TE) {
    const int nv = min(TE, a1 - t0);
    if constexpr (TA) {
      ahead.store(s_geo, s_j, nullptr, tid);
      __syncthreads();
      tile_hidden<TE, kPerTile<MODE, BF>>(W.w1, s_geo, s_hid, tid);
    } else {
      load_tile<TE, kPerTile<MODE, BF>, (MODE == 0 ? -1 : L)>(A.geo, A.a_j, nullptr, t0, nv, i, W.w1, s_geo, s_j, nullptr, s_hid, tid);
    }
    radial_w<L, MODE, C, CB, BF, TE, SWZ>(SWZ && !BF ? W.w2sf[MODE < 3 ? MODE : 0] : W.w2, SWZ && BF ? W.w2sw[MODE < 3 ? MODE : 0] : W.w2b, cbase, s_hid, s_w, wv, lane);
    __syncthreads();
    if constexpr (EF) frame_setup<TE>(s_geo, s_d2, nv, tid);
    if (TA && t0 + TE < a1) ahead.fetch(A.geo, A.a_j, nullptr, t0 + TE, min(TE, a1 - t0 - TE), i, tid);
    // pruned layers gather the sender features of the slot's next edge one iteration
    // ahead (the unpruned ones have no registers to spare for it)
    constexpr bool PF = MODE != 0;
    TF xr[KX];
    if (PF && sl < nv) {
      const int j = s_j[sl];
#pragma unroll
      for (int k = 0; k < KX; ++k) xr[k] = ht[((size_t)j * K + k) * C + cbase + c];
    }
    for (int e = sl; e < nv; e += NS) {
      const float* g = s_geo + e * kGeo;
      const float u = g[G_U];
      float x[K], w[NA], v[K];
      if constexpr (PF) {
#pragma unroll
        for (int k = 0; k < K; ++k) x[k] = k < KX ? to_f(xr[k]) : 0.f;
        if (e + NS < nv) {
          const int j = s_j[e + NS];
#pragma unroll
          for (int k = 0; k < KX; ++k) xr[k] = ht[((size_t)j * K + k) * C + cbase + c];
        }
      } else {
        const int j = s_j[e];
#pragma unroll
        for (int k = 0; k < K; ++k) x[k] = k < KX ? FeatIO<TF>::ld(ht + ((size_t)j * K + k) * C + cbase + c) : 0.f;
      }
#pragma unroll
      for (int k = 0; k < K; ++k) v[k] = 0.f;
      // v is formed with the MLP outputs w'_q; the message is u v (path weights u w'_q)
#pragma unroll
      for (int q = 0; q < NA; ++q) w[q] = FeatIO<WT>::ld(s_w + e * SWE + q * CB + c);
      if constexpr (EF) {
        const float* R = g + G_Y;
        const float* d2 = s_d2 + e * kD2;
        float xp[K], vp[K];
        rot_in<L>(R, d2, x, xp);
#pragma unroll
        for (int k = 0; k < K; ++k) vp[k] = 0.f;
        tpz_fwd<L>(xp, w, vp);
        rot_out_add<L>(R, d2, vp, v);
      } else {
        float Y[K];
#pragma unroll
        for (int k = 0; k < K; ++k) Y[k] = g[G_Y + k];
        tp_fwd<L, MODE>(x, Y, w, v);
      }
      const float av = head_sum<DHC>(qc * (u * v[0]), DH) * rs;
      if (u > 0.f) {
        // the running state is rescaled only when the maximum grows (rarely after the
        // first edges of a row)
        if (av > Mx) {
          const float sc = __expf(Mx - av);
          Zs *= sc;
#pragma unroll
          for (int k = 0; k < KV; ++k) macc[k] *= sc;
          Mx = av;
        }
        const float f = u * __expf(av - Mx);
        Zs += f;
        const float fu = f * u;  // weight of the message u v
#pragma unroll
        for (int k = 0; k < KV; ++k) macc[k] += fu * v[k];
      }
    }
    __syncthreads();
  }
  // merge the NS partial softmax states of every channel
  float* mrg = (float*)s_wb;
  mrg[tid * (KV + 2) + 0] = Mx;
  mrg[tid * (KV + 2) + 1] = Zs;
#pragma unroll
  for (int k = 0; k < KV; ++k) mrg[tid * (KV + 2) + 2 + k] = macc[k];
  __syncthreads();
  if (tid < CB) {
    float M = -INFINITY;
    for (int s = 0; s < NS; ++s) M = fmaxf(M, mrg[(s * CB + tid) * (KV + 2)]);
    float Z = 0.f, mm[KV];
#pragma unroll
    for (int k = 0; k < KV; ++k) mm[k] = 0.f;
    if (M > -INFINITY) {
      for (int s = 0; s < NS; ++s) {
        const float* q = mrg + (s * CB + tid) * (KV + 2);
        const float sc = __expf(q[0] - M);
        Z += q[1] * sc;
#pragma unroll
        for (int k = 0; k < KV; ++k) mm[k] += q[2 + k] * sc;
      }
    }
    const float inv = Z > 0.f ? 1.0f / Z : 0.f;
    // the top layer (MODE & 2) stores only the scalar rows: its node update and node
    // backward read nothing else (the other rows would be zero)
#pragma unroll
    for (int k = 0; k < KV; ++k) FeatIO<TF>::st(m_out + ((size_t)i * K + k) * C + cbase + tid, mm[k] * inv);
    if ((cbase + tid) % DH == 0) {
      const int hd = (cbase + tid) / DH;
      A.mz[((size_t)i * A.heads + hd) * 2 + 0] = M;
      A.mz[((size_t)i * A.heads + hd) * 2 + 1] = Z;
    }
  }
}

// ====================================================================== edge backward, receiver side
// Per row i: recompute w and the tensor product, softmax backward with
// S_i^k = sum_{c in k} g_m_i . m_i (one sweep), gradients w.r.t. q_i, w (-> radial
// MLP -> r), Y (-> rhat) and u; stores alpha and dE/da per edge for the sender pass.
template <int L, int MODE, int C, class TF, int DHC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MODE == 0 ? 4 : (MODE == 1 && sizeof(TF) == 2 ? 6 : 5)))) void k_edge_bwd_recv(EdgeArgs A, LayerW W, BwdArgs B) {
  constexpr int TE = fs_tile_edges<MODE, sizeof(TF) == 2>();
  constexpr int K = Dims<L>::K, NA = Paths<L, MODE>::count();
  constexpr int KX = (MODE & 1) ? 1 : K;
  constexpr int KV = (MODE & 2) ? 1 : K;
  constexpr int CB = fs_channel_block<MODE, sizeof(TF) == 2>(C);
  constexpr int EPW = 64 / CB, NS = kNW * EPW;
  constexpr bool BF = sizeof(TF) == 2;
  constexpr bool SWZ = MODE <= 2 && C >= 32;  // fragment-ordered W_2 copies
  __shared__ __align__(16) float s_geo[TE * kGeo];
  __shared__ int s_j[TE];
  using HT = std::conditional_t<BF, uint16_t, float>;  // hidden units stored as the MFMA reads them
  __shared__ __align__(16) HT s_hid[TE * hid_stride<HT>()];
  __shared__ float s_red[TE * 4];  // per edge: dE/du, dE/drhat (x, y, z), summed over the block's channels
  // w' of the tile, overwritten in place by dE/dw (each element is read, then
  // written, by the same thread)
  using WT = std::conditional_t<BF, uint16_t, float>;
  constexpr int SWE = sw_stride<NA, CB, BF>();
  // the same storage later holds the per-wave partial g_B and the g_q slot sums
  constexpr int SWB = std::max<int>(TE * SWE * sizeof(WT), std::max<int>(kNW * kNB * TE, 256) * sizeof(float));
  __shared__ __align__(16) unsigned char s_wb[SWB];
  WT* s_w = (WT*)s_wb;
  int i, cblk;
  xcd_row_block(i, cblk);
  const int cbase = cblk * CB;
  const int tid = threadIdx.x, wv = MODE == 0 ? tid >> 6 : wave_index(), lane = tid & 63;
  const int slot = lane / CB, c = lane % CB, sl = wv * EPW + slot;
  const int DH = DHC > 0 ? DHC : A.dh;
  const int hd = (cbase + c) / DH;
  const bool lead = ((cbase + c) % DH) == 0;
  const float rs = rsqrtf((float)DH);
  const TF* __restrict__ ht = (const TF*)A.ht;
  const TF* __restrict__ msv = (const TF*)B.m_saved;
  const float qc = A.q[(size_t)i * C + cbase + c];
  float gm[KV], sdot = 0.f;
#pragma unroll
  for (int k = 0; k < KV; ++k) {
    gm[k] = B.g_m[((size_t)i * K + k) * C + cbase + c];
    sdot += gm[k] * FeatIO<TF>::ld(msv + ((size_t)i * K + k) * C + cbase + c);
  }
  const float S = head_sum<DHC>(sdot, DH);
  const float Mi = A.mz[((size_t)i * A.heads + hd) * 2 + 0];
  const float Zi = A.mz[((size_t)i * A.heads + hd) * 2 + 1];
  const float invZ = Zi > 0.f ? 1.0f / Zi : 0.f;
  const float rc = A.rc;
  const float bnorm = sqrtf(2.0f / rc), kpi = 3.14159265358979323846f / rc;
  float gq = 0.f;
  const int a0 = A.abeg[i], a1 = A.aend[i];
  constexpr bool EF = MODE == 0;  // unpruned layers: products in each edge's own frame
  float* s_d2 = (float*)s_hid;    // l = 2 rotation blocks, once the hidden tile is consumed
  static_assert(TE * kD2 * sizeof(float) <= sizeof(s_hid), "rotation blocks fit");
  for (int t0 = a0; t0 < a1; t0 += TE) {
    const int nv = min(TE, a1 - t0);
    load_tile<TE, kPerTile<MODE, BF>, (MODE == 0 ? -1 : L)>(A.geo, A.a_j, nullptr, t0, nv, i, W.w1, s_geo, s_j, nullptr, s_hid, tid);
    radial_w<L, MODE, C, CB, BF, TE, SWZ>(SWZ && !BF ? W.w2sf[MODE < 3 ? MODE : 0] : W.w2, SWZ && BF ? W.w2sw[MODE < 3 ? MODE : 0] : W.w2b, cbase, s_hid, s_w, wv, lane);
    __syncthreads();
    if constexpr (EF) frame_setup<TE>(s_geo, s_d2, nv, tid);
    for (int e = sl; e < nv; e += NS) {
      const float* g = s_geo + e * kGeo;
      const float u = g[G_U];
      const int j = s_j[e];
      float x[K], w[NA], dot[NA], y0[NA];
#pragma unroll
      for (int k = 0; k < K; ++k) x[k] = k < KX ? FeatIO<TF>::ld(ht + ((size_t)j * K + k) * C + cbase + c) : 0.f;
#pragma unroll
      for (int q = 0; q < NA; ++q) w[q] = u * FeatIO<WT>::ld(s_w + e * SWE + q * CB + c);
      // v = sum_q w_q y_q is needed only through v^0 (logit) and g_m . v; in the
      // edge frame x and g_m are rotated (x', g_m') and the products taken at the pole
      float Y[EF ? 1 : K], xp[EF ? K : 1], gmp[EF ? K : 1];
      const float* R = g + G_Y;
      const float* d2 = s_d2 + e * kD2;
      if constexpr (EF) {
        rot_in<L>(R, d2, x, xp);
        rot_in<L>(R, d2, gm, gmp);
        tpz_fwd_dot<L>(xp, gmp, dot, y0);
      } else {
#pragma unroll
        for (int k = 0; k < K; ++k) Y[k] = g[G_Y + k];
        tp_fwd_dot<L, MODE, KV>(x, Y, gm, dot, y0);
      }
      constexpr const cgc::Table& T = cgc::TableOf<L>::t;
      float v0 = 0.f, gdot = 0.f;
#pragma unroll
      for (int q = 0; q < NA; ++q) {
        if (T.p[Paths<L, MODE>::idx(q)].l3 == 0) v0 += w[q] * y0[q];
        gdot += w[q] * dot[q];
      }
      const float av = head_sum<DHC>(qc * v0, DH) * rs;
      const float ghat = head_sum<DHC>(gdot, DH);
      const float beta = __expf(av - Mi) * invZ;
      const float alpha = u * beta;
      const float ga = alpha * (ghat - S);
      const float gqs = ga * qc * rs;
      gq += ga * v0 * rs;
      // dE/dw_q = g_v . y_q with g_v = alpha g_m + e_0 ga q rs; dE/du collects
      // sum_q w'_q dE/dw_q.  The tile keeps dE/dw_q; dE/dw'_q = u dE/dw_q is formed
      // after the W_2^T product, one factor per edge.
      float gwsum = 0.f;
#pragma unroll
      for (int q = 0; q < NA; ++q) {
        float gw = alpha * dot[q];
        if (T.p[Paths<L, MODE>::idx(q)].l3 == 0) gw += gqs * y0[q];
        FeatIO<WT>::st(s_w + e * SWE + q * CB + c, gw);
        gwsum += w[q] * gw;
      }
      float gu = (lead ? beta * (ghat - S) : 0.f) + gwsum * __builtin_amdgcn_rcpf(u);  // u > 0 here; 1-ulp reciprocal
      float grx = 0.f, gry = 0.f, grz = 0.f;
      if constexpr (EF) {
        // tangential dE/drhat along e1, e2 from the pole derivatives; g_v' = alpha g_m' + e_0 ga q rs,
        // taken times u because the product takes w'_q for the path weights u w'_q
        float gvp[K];
#pragma unroll
        for (int k = 0; k < K; ++k) gvp[k] = alpha * gmp[k];
        gvp[0] += gqs;
        tpz_grad_dir<L>(xp, gvp, w, grx, gry);
      } else {
        float gv[K], t[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
          gv[k] = k < KV ? alpha * gm[k] : 0.f;
          t[k] = 0.f;
        }
        gv[0] += gqs;
        tp_grad_y<L, MODE>(x, gv, w, t);
        // dE/dY -> dE/drhat per channel (linear), so only four sums cross the lanes
        real_sh_grad<L>(g[G_RH], g[G_RH + 1], g[G_RH + 2], t, grx, gry, grz);
      }
      // the four channel sums at once; quarter k of the slot's lanes ends with sum k
      const float rsum = gsum4<CB>(gu, grx, gry, grz);
      if (c % (CB / 4) == 0) s_red[e * 4 + c / (CB / 4)] = rsum;
      if (lead) {
        B.ag[((size_t)(t0 + e) * A.heads + hd) * 2 + 0] = alpha;
        B.ag[((size_t)(t0 + e) * A.heads + hd) * 2 + 1] = ga;
      }
    }
    // Padded edges of the last tile contribute nothing to the MLP backward: their
    // geometry rows are zero, so their hidden units (SiLU(0) = 0) and their w' rows are
    // exact zeros, which the edge loop leaves in place of dE/dw.
    constexpr bool PRE = MODE == 0 && BF;  // unpruned bf16 layers: the first W_2^T fragments ahead
    W2tFrags<L, MODE, C, CB, SWZ> fr;
    if constexpr (PRE) fr.fetch(per_tile_global(SWZ ? W.w2tsw[MODE < 3 ? MODE : 0] : W.w2tb), cbase, wv, lane);
    // The recomputed pre-activations (their SiLU' formed in a pass of its own, which
    // spills less in the pruned receivers than forming it inside the W_1^T products)
    // and the W_1^T fragments; forming them before the barrier measured slower.
    constexpr int NEB = TE / 16;
    f4v dpre[NEB];
    const int m = lane & 15, g = lane >> 4;
    float a1t[4];
    auto mlp_in = [&]() {
      radial_pre<TE, kPerTile<MODE, BF>>(W.w1, s_geo, wv, lane, dpre);
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
        for (int r = 0; r < 4; ++r) dpre[eb][r] = dsilu(dpre[eb][r]);
      const float* w1 = per_tile<kPerTile<MODE, BF>>(W.w1);
#pragma unroll
      for (int r = 0; r < 4; ++r) a1t[r] = m < kNB ? w1[(16 * wv + 4 * g + r) * kNB + m] : 0.f;
    };
    __syncthreads();
    // g_s = W_2^T (u * g_w), g_pre = g_s * SiLU'(pre) and g_B = W_1^T g_pre on MFMA:
    // g_s and the recomputed pre-activations share one accumulator layout, and each
    // wave sums g_B over its own 16 hidden units (K index k <-> unit 16 wv + 4k + r).
    {
      f4v gs[NEB], gb[NEB];
      radial_w_bwd<L, MODE, C, CB, BF, TE, SWZ>(SWZ && !BF ? W.w2tsf[MODE < 3 ? MODE : 0] : W.w2t, SWZ && BF ? W.w2tsw[MODE < 3 ? MODE : 0] : W.w2tb, cbase, s_w, gs, wv, lane, PRE ? fr.a : nullptr);
      mlp_in();
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb) {
        gb[eb] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r)
          gb[eb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1t[r], gs[eb][r] * dpre[eb][r], gb[eb], 0, 0, 0);
      }
      __syncthreads();  // every wave is done with the w' tile; its storage takes the partial g_B
      float* s_gb = (float*)s_wb;  // [kNW][kNB][TE]
      if (g < 2) {
#pragma unroll
        for (int eb = 0; eb < NEB; ++eb)
#pragma unroll
          for (int r = 0; r < 4; ++r) s_gb[(wv * kNB + 4 * g + r) * TE + 16 * eb + m] = gb[eb][r];
      }
      __syncthreads();
      // per edge: TPE threads, thread n < 8 takes Bessel function n; dE/dr and dE/dd
      constexpr int TPE = 256 / TE;
      static_assert(TPE >= kNB, "one thread per Bessel function");
      const int e = tid / TPE, q = tid % TPE;
      const float* ge = s_geo + e * kGeo;
      const float r = ge[G_R], ir = 1.0f / r;
      float term = 0.f;
      if (q < kNB) {
        float gBq = 0.f;
#pragma unroll
        for (int w = 0; w < kNW; ++w) gBq += s_gb[(w * kNB + q) * TE + e];
        float sn, cs;
        __sincosf((float)(q + 1) * kpi * r, &sn, &cs);
        // the tile held dE/dw, so the products above give dE/dB / u: dE/dw' = u dE/dw
        term = gBq * ge[G_U] * bnorm * ((float)(q + 1) * kpi * cs * ir - sn * ir * ir);
      }
      term = gsum<TPE>(term);
      if (q < 3 && e < nv) {
        const float gr = s_red[e * 4] * ge[G_DU] + term;
        const float x = ge[G_RH], y = ge[G_RH + 1], z = ge[G_RH + 2];
        const float gx = s_red[e * 4 + 1], gy = s_red[e * 4 + 2], gz = s_red[e * 4 + 3];
        const float rq = q == 0 ? x : (q == 1 ? y : z);
        float tq;  // component q of the tangential part of dE/drhat
        if constexpr (EF) {
          tq = gx * ge[G_Y + q] + gy * ge[G_Y + 3 + q];  // e1, e2 are rows 0 and 1 of R
        } else {
          const float dt = x * gx + y * gy + z * gz;
          tq = (q == 0 ? gx : (q == 1 ? gy : gz)) - dt * rq;
        }
        // one partial per 32-channel slot (C itself below 32), even and odd slots in two
        // arrays of edge-major records; a 64-channel block writes the slot of its first 32
        // channels, and in the first layer's pass (the last receiver pass) it also adds
        // in the odd slot of its second 32 channels, so the force gather reads the even
        // slots only
        const int sl32 = cbase / edge_channel_block(C, BF);
        float* o = B.gd + (((size_t)(sl32 & 1) * B.gd_cap + (t0 + e)) * B.gd_half + (sl32 >> 1)) * 3 + q;
        float val = gr * rq + tq * ir;
        if constexpr (fold_slot_pairs<MODE, BF>(C))
          val += B.gd[(((size_t)B.gd_cap + (t0 + e)) * B.gd_half + (sl32 >> 1)) * 3 + q];
        *o += val;
      }
    }
    __syncthreads();
  }
  // sum g_q over the block's edge slots
  float* sf = (float*)s_wb;
  sf[tid] = gq;
  __syncthreads();
  if (tid < CB) {
    float s = 0.f;
    for (int q = 0; q < NS; ++q) s += sf[q * CB + tid];
    B.g_q[(size_t)i * C + cbase + tid] = s;
  }
}

// ====================================================================== edge backward, sender side
// Per row j: dE/dht_j = sum over edges e = (i <- j) of the transposed tensor
// product, visited as the row's own edges f = (j <- i) with e = arev[f];
// w is symmetric in the pair and Y(-rhat) = (-1)^l Y(rhat).  No atomics.
template <int L, int MODE, int C, class TF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MODE == 0 ? 4 : (sizeof(TF) == 2 ? 7 : 6)))) void k_edge_bwd_send(EdgeArgs A, LayerW W, BwdArgs B) {
  constexpr int TE = fs_tile_edges<MODE, sizeof(TF) == 2>();
  constexpr int K = Dims<L>::K, NA = Paths<L, MODE>::count();
  constexpr int KV = (MODE & 2) ? 1 : K;   // only these components of g_v can be nonzero
  constexpr int KX = (MODE & 1) ? 1 : K;   // only these input gradients are needed
  constexpr int CB = fs_channel_block<MODE, sizeof(TF) == 2>(C);
  constexpr int EPW = 64 / CB, NS = kNW * EPW;
  constexpr bool BF = sizeof(TF) == 2;
  constexpr bool SWZ = MODE <= 2 && C >= 32;  // fragment-ordered W_2 copies
  __shared__ __align__(16) float s_geo[TE * kGeo];
  __shared__ int s_j[TE];
  __shared__ int s_ae[TE];
  using HT = std::conditional_t<BF, uint16_t, float>;  // hidden units stored as the MFMA reads them
  __shared__ __align__(16) HT s_hid[TE * hid_stride<HT>()];
  using WT = std::conditional_t<BF, uint16_t, float>;
  constexpr int SWE = sw_stride<NA, CB, BF>();
  constexpr int SWB = std::max<int>(TE * SWE * sizeof(WT), 256 * KX * sizeof(float));
  __shared__ __align__(16) unsigned char s_wb[SWB];
  WT* s_w = (WT*)s_wb;
  int jrow, cblk;
  xcd_row_block(jrow, cblk);
  const int cbase = cblk * CB;
  const int tid = threadIdx.x, wv = MODE == 0 ? tid >> 6 : wave_index(), lane = tid & 63;
  const int slot = lane / CB, c = lane % CB, sl = wv * EPW + slot;
  const int DH = A.dh;
  const int hd = (cbase + c) / DH;
  const float rs = rsqrtf((float)DH);
  float acc[K];
#pragma unroll
  for (int k = 0; k < K; ++k) acc[k] = 0.f;
  const int a0 = A.abeg[jrow], a1 = A.aend[jrow];
  constexpr bool EF = MODE == 0;  // unpruned layers: products in each edge's own frame
  float* s_d2 = (float*)s_hid;    // l = 2 rotation blocks, once the hidden tile is consumed
  static_assert(TE * kD2 * sizeof(float) <= sizeof(s_hid), "rotation blocks fit");
  // unpruned layers gather the next tile's geometry during the current tile
  constexpr bool TA = MODE == 0;
  TileAhead<TE, true> ahead;
  if (TA && a0 < a1) ahead.fetch(A.geo, A.a_j, A.arev, a0, min(TE, a1 - a0), jrow, tid);
  for (int t0 = a0; t0 < a1; t0 += TE) {
    const int nv = min(TE, a1 - t0);
    if constexpr (TA) {
      ahead.store(s_geo, s_j, s_ae, tid);
      __syncthreads();
      tile_hidden<TE, kPerTile<MODE, BF>>(W.w1, s_geo, s_hid, tid);
    } else {
      load_tile<TE, kPerTile<MODE, BF>, (MODE == 0 ? -1 : L)>(A.geo, A.a_j, A.arev, t0, nv, jrow, W.w1, s_geo, s_j, s_ae, s_hid, tid);
    }
    radial_w<L, MODE, C, CB, BF, TE, SWZ>(SWZ && !BF ? W.w2sf[MODE < 3 ? MODE : 0] : W.w2, SWZ && BF ? W.w2sw[MODE < 3 ? MODE : 0] : W.w2b, cbase, s_hid, s_w, wv, lane);
    __syncthreads();
    if constexpr (EF) frame_setup<TE, true>(s_geo, s_d2, nv, tid);
    if (TA && t0 + TE < a1) ahead.fetch(A.geo, A.a_j, A.arev, t0 + TE, min(TE, a1 - t0 - TE), jrow, tid);
    // the receiver-side data of the slot's next edge are gathered one iteration ahead
    float gmr[KV], agr[2], qr = 0.f;
    auto gather = [&](int f) {
      const int irow = s_j[f];
      const int e = s_ae[f];
      agr[0] = B.ag[((size_t)e * A.heads + hd) * 2 + 0];
      agr[1] = B.ag[((size_t)e * A.heads + hd) * 2 + 1];
      qr = A.q[(size_t)irow * C + cbase + c];
#pragma unroll
      for (int k = 0; k < KV; ++k) gmr[k] = B.g_m[((size_t)irow * K + k) * C + cbase + c];
    };
    if (sl < nv) gather(sl);
    for (int f = sl; f < nv; f += NS) {
      const float* g = s_geo + f * kGeo;
      const float u = g[G_U];
      // the products take the MLP outputs w'_q for the path weights u w'_q, so g_v enters
      // times u
      const float au = agr[0] * u;
      float gv[K], w[NA];
#pragma unroll
      for (int k = 0; k < K; ++k) gv[k] = k < KV ? au * gmr[k] : 0.f;
      gv[0] += agr[1] * qr * rs * u;
      if (f + NS < nv) gather(f + NS);
#pragma unroll
      for (int q = 0; q < NA; ++q) w[q] = FeatIO<WT>::ld(s_w + f * SWE + q * CB + c);
      if constexpr (EF) {
        // in f's frame the edge e points along -z-hat
        const float* R = g + G_Y;
        const float* d2 = s_d2 + f * kD2;
        float gvp[K], gxp[K];
        rot_in<L>(R, d2, gv, gvp);
#pragma unroll
        for (int k = 0; k < K; ++k) gxp[k] = 0.f;
        tpz_grad_x<L, true>(gvp, w, gxp);
        rot_out_add<L>(R, d2, gxp, acc);
      } else {
        float Y[K];
#pragma unroll
        for (int l = 0; l <= L; ++l)
#pragma unroll
          for (int mm = 0; mm < 2 * l + 1; ++mm) Y[l * l + mm] = (l & 1) ? -g[G_Y + l * l + mm] : g[G_Y + l * l + mm];
        tp_grad_x<L, MODE>(Y, gv, w, acc);
      }
    }
    __syncthreads();
  }
  float* mrg = (float*)s_wb;
#pragma unroll
  for (int k = 0; k < KX; ++k) mrg[tid * KX + k] = acc[k];
  __syncthreads();
  if (tid < CB) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      float s = 0.f;
      if (k < KX)
        for (int q = 0; q < NS; ++q) s += mrg[(q * CB + tid) * KX + k];
      B.g_ht[((size_t)jrow * K + k) * C + cbase + tid] = s;
    }
  }
}

// ====================================================================== forces
// F_k = sum_{a in row k} (dE/dd_a - dE/dd_{arev[a]}), un-permuted; one wave per row,
// lanes over the row's active edges, then a wave sum.  dE/dd of an edge is the sum of
// its HS even-slot partials and, unless the last receiver pass folded them in (ODD =
// false), its HS odd-slot partials: edge-major records [HS][3] in each half.
template <int HS, bool ODD>
__device__ __forceinline__ void grad_record(const float* __restrict__ gd, size_t half, int a, float& x, float& y,
                                            float& z) {
  const float* r = gd + (size_t)a * (3 * HS);
  if constexpr (HS == 2) {
    const f4v u = *(const f4v*)r;
    const float2 v = *(const float2*)(r + 4);
    x = u[0] + u[3];
    y = u[1] + v.x;
    z = u[2] + v.y;
  } else {
    x = r[0];
    y = r[1];
    z = r[2];
  }
  if constexpr (ODD) {
    float ox, oy, oz;
    grad_record<HS, false>(gd + half, 0, a, ox, oy, oz);
    x += ox;
    y += oy;
    z += oz;
  }
}

template <int HS, bool ODD>
__global__ __launch_bounds__(256) void k_forces(const int32_t* __restrict__ abeg, const int32_t* __restrict__ aend,
                                                const int32_t* __restrict__ arev, const float* __restrict__ gd,
                                                int64_t cap, int n, const int32_t* __restrict__ perm,
                                                float* __restrict__ F, int32_t* __restrict__ flag) {
  const int k = row_block0() + wave_index(), lane = threadIdx.x & 63;
  if (k >= n) return;
  const size_t half = (size_t)cap * 3 * HS;  // floats from an even-slot record to the odd one
  float fx = 0.f, fy = 0.f, fz = 0.f;
  for (int a = abeg[k] + lane; a < aend[k]; a += 64) {
    float ax, ay, az, bx, by, bz;
    grad_record<HS, ODD>(gd, half, a, ax, ay, az);
    grad_record<HS, ODD>(gd, half, arev[a], bx, by, bz);
    fx += ax - bx;
    fy += ay - by;
    fz += az - bz;
  }
  fx = wave_sum(fx);
  fy = wave_sum(fy);
  fz = wave_sum(fz);
  if (lane == 0) {
    const int o = perm ? perm[k] : k;
    F[3 * o + 0] = fx;
    F[3 * o + 1] = fy;
    F[3 * o + 2] = fz;
    if (!isfinite(fx) || !isfinite(fy) || !isfinite(fz)) atomicOr(flag, 1);
  }
}

__global__ void k_check_energy(const double* e, int32_t* flag) {
  if (!isfinite(e[0])) atomicOr(flag, 1);
}

// weighted sum of the heads' energies, float64, in head order (one thread)
__global__ void k_weighted_sum(const double* __restrict__ e, const float* __restrict__ lam, int R, double* out,
                               int32_t* flag) {
  double s = 0.0;
  for (int k = 0; k < R; ++k) s += (double)lam[k] * e[k];
  out[0] = s;
  if (!isfinite(s)) atomicOr(flag, 1);
}

// ====================================================================== dispatch
template <int L, int C, class TF>
struct Launch {
  template <int MODE>
  static void edge_fwd(const Plan& P, const EdgeArgs& a, const LayerW& W, void* m, hipStream_t st) {
    constexpr int CB = fs_channel_block<MODE, sizeof(TF) == 2>(C);
    static const char* names[4] = {"edge_fwd", "edge_fwd_first", "edge_fwd_last", "edge_fwd_single"};
    ProfScope ps(names[MODE], st);
    // heads of 32 channels (the common configuration) get straight-line head sums
    if (C >= 32 && a.dh == 32)
      k_edge_fwd<L, MODE, C, TF, (C >= 32 ? 32 : 0)><<<dim3(P.n, C / CB), 256, 0, st>>>(a, W, (TF*)m);
    else
      k_edge_fwd<L, MODE, C, TF, 0><<<dim3(P.n, C / CB), 256, 0, st>>>(a, W, (TF*)m);
  }
  template <int MODE>
  static void edge_bwd(const Plan& P, const EdgeArgs& A, const LayerW& W, const BwdArgs& B, bool input_grad,
                       hipStream_t st) {
    constexpr int CB = fs_channel_block<MODE, sizeof(TF) == 2>(C);
    static const char* rn[4] = {"edge_bwd_recv", "edge_bwd_recv_first", "edge_bwd_recv_last", "edge_bwd_recv_single"};
    static const char* sn[4] = {"edge_bwd_send", "edge_bwd_send_first", "edge_bwd_send_last", "edge_bwd_send_single"};
    {
      ProfScope ps(rn[MODE], st);
      if (C >= 32 && A.dh == 32)
        k_edge_bwd_recv<L, MODE, C, TF, (C >= 32 ? 32 : 0)><<<dim3(P.n, C / CB), 256, 0, st>>>(A, W, B);
      else
        k_edge_bwd_recv<L, MODE, C, TF, 0><<<dim3(P.n, C / CB), 256, 0, st>>>(A, W, B);
    }
    if (input_grad) {
      ProfScope ps(sn[MODE], st);
      k_edge_bwd_send<L, MODE, C, TF><<<dim3(P.n, C / fs_channel_block<MODE, sizeof(TF) == 2>(C)), 256, 0, st>>>(A, W, B);
    }
  }
  static int layer_fwd(const Plan& P, const EdgeArgs& A, const LayerW& W, const void* h_in, void* h_out,
                       void* ht, float* q, void* m, int mode, hipStream_t st) {
    const int n = P.n;
    const int nblk = (int)cdiv(n, kNAT);
    if (mode & 1)
      k_pre_linear<L, C, TF, true><<<nblk, atom_waves<C>() * 64, 0, st>>>((const TF*)h_in, n, W, (TF*)ht, q);
    else
      k_pre_linear<L, C, TF><<<nblk, atom_waves<C>() * 64, 0, st>>>((const TF*)h_in, n, W, (TF*)ht, q);
    EdgeArgs a = A;
    a.ht = ht;
    a.q = q;
    switch (mode) {
      case 1: edge_fwd<1>(P, a, W, m, st); break;
      case 2: edge_fwd<2>(P, a, W, m, st); break;
      case 3: edge_fwd<3>(P, a, W, m, st); break;
      default: edge_fwd<0>(P, a, W, m, st); break;
    }
    if (mode & 2)
      k_node_update<L, C, TF, true><<<nblk, atom_waves<C>() * 64, 0, st>>>((const TF*)m, (const TF*)h_in, n, W,
                                                                            (TF*)h_out);
    else if (mode & 1)
      k_node_update<L, C, TF, false, true><<<nblk, atom_waves<C>() * 64, 0, st>>>((const TF*)m, (const TF*)h_in, n,
                                                                                  W, (TF*)h_out);
    else
      k_node_update<L, C, TF><<<nblk, atom_waves<C>() * 64, 0, st>>>((const TF*)m, (const TF*)h_in, n, W, (TF*)h_out);
    MP_CHECK_LAUNCH();
    return MP_OK;
  }
  static int embed(const Plan& P, const float* emb, const int32_t* sp, void* h, bool zero_rows, hipStream_t st) {
    constexpr int K = Dims<L>::K;
    const int64_t tot = (int64_t)P.n * (C / 8);
    if (zero_rows)
      k_embed<K, C, TF><<<cdiv(tot, 256), 256, 0, st>>>(emb, sp, P.n, (TF*)h);
    else
      k_embed<K, C, TF, false><<<cdiv(tot, 256), 256, 0, st>>>(emb, sp, P.n, (TF*)h);
    MP_CHECK_LAUNCH();
    return MP_OK;
  }
  static int readout(const Plan& P, int R, const void* h, const float* wrT, const float* wout, float* e_atoms,
                     hipStream_t st) {
    k_readout<C, TF><<<cdiv(P.n, kAPB), C, 0, st>>>((const TF*)h, P.n, Dims<L>::K, R, wrT, wout, e_atoms);
    MP_CHECK_LAUNCH();
    return MP_OK;
  }
  static int readout_bwd(const Plan& P, int R, const void* h, const float* wrT, const float* wr, const float* wout,
                         const float* lam, float* g_h, hipStream_t st) {
    k_readout_bwd<C, TF><<<cdiv(P.n, kAPB), C, 0, st>>>((const TF*)h, P.n, Dims<L>::K, R, wrT, wr, wout, lam,
                                                        g_h);
    MP_CHECK_LAUNCH();
    return MP_OK;
  }
  // input_grad = false (the first layer, whose input is the position-independent
  // embedding): the gradient with respect to the layer's input features reaches no
  // force, so the sender pass and the pre-linear backward are not run.
  static int layer_bwd(const Plan& P, const EdgeArgs& A, const LayerW& W, const BwdArgs& B, float* g_h, int mode,
                       bool input_grad, hipStream_t st) {
    const int n = P.n;
    const int nblk = (int)cdiv(n, kNAT);
    if (mode & 2)
      k_node_bwd<L, C, TF, true><<<nblk, atom_waves<C>() * 64, 0, st>>>((const TF*)B.m_saved, g_h, n, W, B.g_m);
    else
      k_node_bwd<L, C, TF><<<nblk, atom_waves<C>() * 64, 0, st>>>((const TF*)B.m_saved, g_h, n, W, B.g_m);
    switch (mode) {
      case 1: edge_bwd<1>(P, A, W, B, input_grad, st); break;
      case 2: edge_bwd<2>(P, A, W, B, input_grad, st); break;
      case 3: edge_bwd<3>(P, A, W, B, input_grad, st); break;
      default: edge_bwd<0>(P, A, W, B, input_grad, st); break;
    }
    if (input_grad && (mode & 2))
      k_pre_linear_bwd<L, C, TF, true><<<nblk, atom_waves<C>() * 64, 0, st>>>(B.g_ht, B.g_q, n, W, g_h);
    else if (input_grad)
      k_pre_linear_bwd<L, C, TF><<<nblk, atom_waves<C>() * 64, 0, st>>>(B.g_ht, B.g_q, n, W, g_h);
    MP_CHECK_LAUNCH();
    return MP_OK;
  }
};

int geometry(const Plan& P, const mp_graph* g, float rc, Geo& G, hipStream_t st) {
  ProfScope ps("geometry", st);
  const int n = P.n, T = 256;
  const int nb = (int)cdiv(n, kRowsPerBlock);
  k_active_fill<<<nb, T, 0, st>>>(g->pos, g->row_ptr, g->col, g->rev, n, g->box_L, rc, G.aend, G.a_j, G.a_r, G.amap,
                                  G.geo);
  MP_CHECK_LAUNCH();
  k_arev<<<nb, T, 0, st>>>(G.a_r, G.amap, g->row_ptr, G.aend, n, G.arev);
  MP_CHECK_LAUNCH();
  return MP_OK;
}

int launch_forces(const Plan& P, const mp_graph* g, const Geo& G, const float* gd, const int32_t* perm, float* F,
                  int32_t* flag, hipStream_t st) {
  ProfScope ps("forces", st);
  const int nb = (int)cdiv(P.n, kRowsPerBlock);
  const int hs = gd_half_slots(P);
  // the odd slots were folded into the even ones by the first layer's receiver pass when
  // its blocks span two slots (bf16 features, C >= 64); a single slot has no odd partner
  const bool odd = P.ncb > 1 && !(P.bf16 ? fold_slot_pairs<1, true>(P.C) : fold_slot_pairs<1, false>(P.C));
  if (hs == 2 && odd)
    k_forces<2, true><<<nb, 256, 0, st>>>(g->row_ptr, G.aend, G.arev, gd, P.cap, P.n, perm, F, flag);
  else if (hs == 2)
    k_forces<2, false><<<nb, 256, 0, st>>>(g->row_ptr, G.aend, G.arev, gd, P.cap, P.n, perm, F, flag);
  else if (hs == 1 && odd)
    k_forces<1, true><<<nb, 256, 0, st>>>(g->row_ptr, G.aend, G.arev, gd, P.cap, P.n, perm, F, flag);
  else if (hs == 1)
    k_forces<1, false><<<nb, 256, 0, st>>>(g->row_ptr, G.aend, G.arev, gd, P.cap, P.n, perm, F, flag);
  else
    return arg_error("force gather: unsupported number of channel blocks");
  MP_CHECK_LAUNCH();
  return MP_OK;
}

int launch_energy(const float* e_atoms, int n, double* out, int32_t* flag, hipStream_t st) {
  k_energy_sum<<<1, 1024, 0, st>>>(e_atoms, n, out);
  k_check_energy<<<1, 1, 0, st>>>(out, flag);
  MP_CHECK_LAUNCH();
  return MP_OK;
}

int launch_weighted_sum(const double* e, const float* lam, int R, double* out, int32_t* flag, hipStream_t st) {
  k_weighted_sum<<<1, 1, 0, st>>>(e, lam, R, out, flag);
  MP_CHECK_LAUNCH();
  return MP_OK;
}

#define MP_DISPATCH(P, CALL)                                                              \
  do {                                                                                    \
    if ((P).lmax == 1 && (P).C == 16 && !(P).bf16) return Launch<1, 16, float>::CALL;     \
    if ((P).lmax == 2 && (P).C == 16 && !(P).bf16) return Launch<2, 16, float>::CALL;     \
    if ((P).lmax == 2 && (P).C == 64 && !(P).bf16) return Launch<2, 64, float>::CALL;     \
    if ((P).lmax == 2 && (P).C == 128 && !(P).bf16) return Launch<2, 128, float>::CALL;   \
    if ((P).lmax == 2 && (P).C == 128 && (P).bf16) return Launch<2, 128, uint16_t>::CALL; \
    if ((P).lmax == 2 && (P).C == 64 && (P).bf16) return Launch<2, 64, uint16_t>::CALL;   \
    if ((P).lmax == 1 && (P).C == 64 && !(P).bf16) return Launch<1, 64, float>::CALL;     \
    return arg_error("unsupported (lmax, channels, dtype) combination");                  \
  } while (0)

int dispatch_layer_fwd(const Plan& P, const EdgeArgs& A, const LayerW& W, const void* h_in, void* h_out,
                       void* ht, float* q, void* m, int mode, hipStream_t st) {
  MP_DISPATCH(P, layer_fwd(P, A, W, h_in, h_out, ht, q, m, mode, st));
}
int dispatch_embed(const Plan& P, const float* emb, const int32_t* sp, void* h, bool zero_rows, hipStream_t st) {
  MP_DISPATCH(P, embed(P, emb, sp, h, zero_rows, st));
}
int dispatch_readout(const Plan& P, int R, const void* h, const float* wrT, const float* wout, float* e_atoms,
                     hipStream_t st) {
  MP_DISPATCH(P, readout(P, R, h, wrT, wout, e_atoms, st));
}
int dispatch_readout_bwd(const Plan& P, int R, const void* h, const float* wrT, const float* wr, const float* wout,
                         const float* lam, float* g_h, hipStream_t st) {
  MP_DISPATCH(P, readout_bwd(P, R, h, wrT, wr, wout, lam, g_h, st));
}
int dispatch_layer_bwd(const Plan& P, const EdgeArgs& A, const LayerW& W, const BwdArgs& B, float* g_h, int mode,
                       bool input_grad, hipStream_t st) {
  MP_DISPATCH(P, layer_bwd(P, A, W, B, g_h, mode, input_grad, st));
}

__global__ void k_fill_zero(uint32_t* __restrict__ p, int64_t nwords) {
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < nwords; x += (int64_t)gridDim.x * blockDim.x)
    p[x] = 0u;
}

// zero-fill as a kernel (graph-capturable; bytes must be a multiple of 4)
int fill_zero(void* p, size_t bytes, hipStream_t st) {
  const int64_t nw = (int64_t)(bytes / 4);
  const int64_t blocks = std::min<int64_t>(cdiv(nw, 256), 65536);
  k_fill_zero<<<(unsigned)std::max<int64_t>(blocks, 1), 256, 0, st>>>((uint32_t*)p, nw);
  MP_CHECK_LAUNCH();
  return MP_OK;
}

bool supported(int lmax, int C, bool bf16) {
  return (lmax == 1 && C == 16 && !bf16) || (lmax == 2 && C == 16 && !bf16) || (lmax == 2 && C == 64) ||
         (lmax == 2 && C == 128) || (lmax == 1 && C == 64 && !bf16);
}

}  // namespace mdmp
