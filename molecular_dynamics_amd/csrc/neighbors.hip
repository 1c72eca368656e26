// Neighbour build: wrap, Hilbert sort, cell list, skin-padded radius graph.
//
// "Ab Initio Accuracy Beyond the Cutoff" (Abstract): atoms are sorted along a
// space-filling curve, a conservative skin keeps the topology valid between
// rebuilds, and the neighbour search has three levels.  The levels here are
// the Hilbert order itself (rows of nearby atoms are nearby in memory), a
// cell list of side >= r_c + skin, and the exact float64 pair test.  Every
// decision is taken in float64 with contraction off so that the sorted CSR is
// identical bit for bit to the plain statement of the rules in mdmp.h.
#include <climits>

#include "common.hpp"
#include "prof.hpp"

#pragma clang fp contract(off)

namespace mdmp {
namespace nb {

constexpr int kMaxRow = 1024;  // neighbours per row held in LDS while sorting

// Skilling, "Programming the Hilbert curve" (AIP Conf. Proc. 707, 2004):
// transpose form of the Hilbert index for 3 axes, 10 bits each, then the
// transposed bits read out level by level, axis 0 (x) most significant.
__device__ __forceinline__ uint32_t hilbert30(uint32_t x0, uint32_t x1, uint32_t x2) {
  uint32_t X[3] = {x0, x1, x2};
  const uint32_t top = 1u << 9;
  for (uint32_t q = top; q > 1; q >>= 1) {
    const uint32_t low = q - 1;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      if (X[i] & q) {
        X[0] ^= low;
      } else {
        uint32_t t = (X[0] ^ X[i]) & low;
        X[0] ^= t;
        X[i] ^= t;
      }
    }
  }
  X[1] ^= X[0];
  X[2] ^= X[1];
  uint32_t t = 0;
  for (uint32_t q = top; q > 1; q >>= 1)
    if (X[2] & q) t ^= q - 1;
  X[0] ^= t;
  X[1] ^= t;
  X[2] ^= t;
  uint32_t key = 0;
  for (int lev = 9; lev >= 0; --lev) {
    key = (key << 1) | ((X[0] >> lev) & 1u);
    key = (key << 1) | ((X[1] >> lev) & 1u);
    key = (key << 1) | ((X[2] >> lev) & 1u);
  }
  return key;
}

// Morton (Z-order) index: the bits of the three 10-bit cell coordinates interleaved,
// most significant level first, x most significant within a level.
__device__ __forceinline__ uint32_t morton30(uint32_t x0, uint32_t x1, uint32_t x2) {
  uint32_t key = 0;
  for (int lev = 9; lev >= 0; --lev) {
    key = (key << 1) | ((x0 >> lev) & 1u);
    key = (key << 1) | ((x1 >> lev) & 1u);
    key = (key << 1) | ((x2 >> lev) & 1u);
  }
  return key;
}

// order: MP_ORDER_HILBERT, MP_ORDER_MORTON, or MP_ORDER_INPUT (every key 0: the stable
// sort keeps the input order)
__global__ void k_wrap_key(const float* __restrict__ pos, int n, float Lf, int order, float* __restrict__ pos_w,
                           uint32_t* __restrict__ key, int32_t* __restrict__ idx) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const double Ld = (double)Lf;
  const double S = 1024.0 / Ld;
  uint32_t g[3];
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    double x = (double)pos[3 * i + a];
    double fl = floor(x / Ld);
    double sh = Ld * fl;
    double w = x - sh;
    if (w < 0.0) w += Ld;
    if (w >= Ld) w -= Ld;
    float f = (float)w;
    if (f >= Lf) f = 0.0f;
    pos_w[3 * i + a] = f;
    double c = floor((double)f * S);
    if (c > 1023.0) c = 1023.0;
    g[a] = (uint32_t)c;
  }
  key[i] = order == MP_ORDER_HILBERT ? hilbert30(g[0], g[1], g[2])
                                     : (order == MP_ORDER_MORTON ? morton30(g[0], g[1], g[2]) : 0u);
  idx[i] = i;
}

// ---------------------------------------------------------------- radix sort
constexpr int kRsThreads = 256;
constexpr int kRsItems = 16;
constexpr int kRsTile = kRsThreads * kRsItems;

__global__ __launch_bounds__(kRsThreads) void k_radix_hist(const uint32_t* __restrict__ keys, int n,
                                                             int shift, int32_t* __restrict__ hist,
                                                             int ntiles) {
  __shared__ int cnt[256];
  const int tid = threadIdx.x;
  cnt[tid] = 0;
  __syncthreads();
  const int base = blockIdx.x * kRsTile;
  for (int i = tid; i < kRsTile; i += kRsThreads) {
    int g = base + i;
    if (g < n) atomicAdd(&cnt[(keys[g] >> shift) & 255u], 1);
  }
  __syncthreads();
  hist[tid * ntiles + blockIdx.x] = cnt[tid];
}

// stable scatter: within a tile, elements keep their order among equal digits
__global__ __launch_bounds__(kRsThreads) void k_radix_scatter(const uint32_t* __restrict__ kin,
                                                                const int32_t* __restrict__ vin,
                                                                uint32_t* __restrict__ kout,
                                                                int32_t* __restrict__ vout, int n,
                                                                int shift,
                                                                const int32_t* __restrict__ offs,
                                                                int ntiles) {
  __shared__ int run[256];
  __shared__ int wcnt[4][256];
  __shared__ int base_off[256];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  run[tid] = 0;
  base_off[tid] = offs[tid * ntiles + blockIdx.x];
#pragma unroll
  for (int q = 0; q < 4; ++q) wcnt[q][tid] = 0;
  __syncthreads();
  for (int r = 0; r < kRsItems; ++r) {
    const int g = blockIdx.x * kRsTile + r * kRsThreads + tid;
    const bool valid = g < n;
    const uint32_t k = valid ? kin[g] : 0u;
    const int d = (int)((k >> shift) & 255u);
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      uint64_t bb = __ballot(valid && ((d >> b) & 1));
      m &= ((d >> b) & 1) ? bb : ~bb;
    }
    const int rank = __popcll(m & ((1ull << lane) - 1ull));
    if (valid && rank == 0) wcnt[w][d] = __popcll(m);
    __syncthreads();
    if (valid) {
      int off = base_off[d] + run[d] + rank;
      for (int q = 0; q < w; ++q) off += wcnt[q][d];
      kout[off] = k;
      vout[off] = vin[g];
    }
    __syncthreads();
    run[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
#pragma unroll
    for (int q = 0; q < 4; ++q) wcnt[q][tid] = 0;
    __syncthreads();
  }
}

// --------------------------------------------------------------------- scan
constexpr int kScThreads = 256;
constexpr int kScItems = 4;
constexpr int kScBlock = kScThreads * kScItems;

__device__ __forceinline__ int64_t block_excl_scan(int64_t v, int64_t* sh, int64_t* total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int o = 1; o < kScThreads; o <<= 1) {
    int64_t t = tid >= o ? sh[tid - o] : 0;
    __syncthreads();
    sh[tid] += t;
    __syncthreads();
  }
  int64_t incl = sh[tid];
  *total = sh[kScThreads - 1];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(kScThreads) void k_scan_sums(const int32_t* __restrict__ in, int64_t n,
                                                            int64_t* __restrict__ bsum) {
  __shared__ int64_t sh[kScThreads];
  const int64_t base = (int64_t)blockIdx.x * kScBlock;
  int64_t s = 0;
  for (int q = 0; q < kScItems; ++q) {
    int64_t g = base + threadIdx.x * kScItems + q;
    if (g < n) s += in[g];
  }
  int64_t tot;
  block_excl_scan(s, sh, &tot);
  if (threadIdx.x == 0) bsum[blockIdx.x] = tot;
}

__global__ __launch_bounds__(kScThreads) void k_scan_partials(int64_t* __restrict__ bsum, int nb,
                                                                int64_t* __restrict__ total) {
  __shared__ int64_t sh[kScThreads];
  int64_t carry = 0;
  for (int base = 0; base < nb; base += kScThreads) {
    int i = base + threadIdx.x;
    int64_t v = i < nb ? bsum[i] : 0;
    int64_t tot;
    int64_t ex = block_excl_scan(v, sh, &tot);
    if (i < nb) bsum[i] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) *total = carry;
}

__global__ __launch_bounds__(kScThreads) void k_scan_apply(const int32_t* __restrict__ in, int64_t n,
                                                             const int64_t* __restrict__ bsum,
                                                             int32_t* __restrict__ out,
                                                             const int64_t* __restrict__ total,
                                                             int write_total) {
  __shared__ int64_t sh[kScThreads];
  const int64_t base = (int64_t)blockIdx.x * kScBlock;
  int64_t vals[kScItems];
  int64_t s = 0;
  for (int q = 0; q < kScItems; ++q) {
    int64_t g = base + threadIdx.x * kScItems + q;
    vals[q] = g < n ? in[g] : 0;
    s += vals[q];
  }
  int64_t tot;
  int64_t ex = block_excl_scan(s, sh, &tot) + bsum[blockIdx.x];
  for (int q = 0; q < kScItems; ++q) {
    int64_t g = base + threadIdx.x * kScItems + q;
    if (g < n) out[g] = (int32_t)ex;
    ex += vals[q];
  }
  if (write_total && blockIdx.x == 0 && threadIdx.x == 0) out[n] = (int32_t)*total;
}

// ----------------------------------------------------------------- gathers
__global__ void k_gather_sorted(const int32_t* __restrict__ perm, const float* __restrict__ pos_w,
                                const int32_t* __restrict__ species, int n, float* __restrict__ pos_s,
                                int32_t* __restrict__ sp_s) {
  int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= n) return;
  int i = perm[s];
  pos_s[3 * s + 0] = pos_w[3 * i + 0];
  pos_s[3 * s + 1] = pos_w[3 * i + 1];
  pos_s[3 * s + 2] = pos_w[3 * i + 2];
  sp_s[s] = species[i];
}

// --------------------------------------------------------------- cell list
__device__ __forceinline__ int cell_coord(float x, double inv_side, int nc) {
  int c = (int)floor((double)x * inv_side);
  return c < 0 ? 0 : (c >= nc ? nc - 1 : c);
}

__global__ void k_cell_id(const float* __restrict__ ps, int n, double inv_side, int nc,
                          uint32_t* __restrict__ cid, int32_t* __restrict__ idx) {
  int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= n) return;
  int cx = cell_coord(ps[3 * s + 0], inv_side, nc);
  int cy = cell_coord(ps[3 * s + 1], inv_side, nc);
  int cz = cell_coord(ps[3 * s + 2], inv_side, nc);
  cid[s] = (uint32_t)((cx * nc + cy) * nc + cz);
  idx[s] = s;
}

__global__ void k_cell_start(const uint32_t* __restrict__ sorted_cid, int n, int ncell,
                             int32_t* __restrict__ cell_start) {
  int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c > ncell) return;
  int lo = 0, hi = n;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (sorted_cid[mid] < (uint32_t)c) lo = mid + 1;
    else hi = mid;
  }
  cell_start[c] = lo;
}

struct PairCtx {
  double L, half, R2;
};

// float64 minimum-image test with the fixed operation order of mdmp.h
__device__ __forceinline__ bool pair_in(double sx, double sy, double sz, const float* __restrict__ pt,
                                        const PairCtx& p) {
  double d0 = (double)pt[0] - sx;
  double d1 = (double)pt[1] - sy;
  double d2 = (double)pt[2] - sz;
  if (d0 > p.half) d0 -= p.L; else if (d0 < -p.half) d0 += p.L;
  if (d1 > p.half) d1 -= p.L; else if (d1 < -p.half) d1 += p.L;
  if (d2 > p.half) d2 -= p.L; else if (d2 < -p.half) d2 += p.L;
  double a = d0 * d0;
  double b = d1 * d1;
  double c = d2 * d2;
  double D = (a + b) + c;
  return D < p.R2;
}

// degree per row; nc == 0 selects the all-pairs test
__global__ void k_count(const float* __restrict__ ps, int n, PairCtx pc, double inv_side, int nc,
                        const int32_t* __restrict__ cell_start, const int32_t* __restrict__ cell_atoms,
                        int32_t* __restrict__ deg, int32_t* __restrict__ flag) {
  int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= n) return;
  const double sx = ps[3 * s], sy = ps[3 * s + 1], sz = ps[3 * s + 2];
  int cnt = 0;
  if (nc == 0) {
    for (int t = 0; t < n; ++t)
      if (t != s && pair_in(sx, sy, sz, ps + 3 * t, pc)) cnt++;
  } else {
    // per (dx, dy): the cells cz-1 .. cz+1 are one run of cell_atoms unless they wrap in z,
    // then two runs (nc >= 3: no cell twice)
    const int cx = cell_coord(ps[3 * s], inv_side, nc), cy = cell_coord(ps[3 * s + 1], inv_side, nc),
              cz = cell_coord(ps[3 * s + 2], inv_side, nc);
    const int lo = cz > 0 ? cz - 1 : 0, hi = cz + 2 < nc ? cz + 2 : nc;
    const int w = cz == 0 ? nc - 1 : (cz == nc - 1 ? 0 : -1);
    for (int dx = -1; dx <= 1; ++dx)
      for (int dy = -1; dy <= 1; ++dy) {
        int ix = cx + dx, iy = cy + dy;
        ix += ix < 0 ? nc : (ix >= nc ? -nc : 0);
        iy += iy < 0 ? nc : (iy >= nc ? -nc : 0);
        const int base = (ix * nc + iy) * nc;
        for (int q = cell_start[base + lo]; q < cell_start[base + hi]; ++q) {
          int t = cell_atoms[q];
          if (t != s && pair_in(sx, sy, sz, ps + 3 * t, pc)) cnt++;
        }
        if (w >= 0)
          for (int q = cell_start[base + w]; q < cell_start[base + w + 1]; ++q) {
            int t = cell_atoms[q];
            if (t != s && pair_in(sx, sy, sz, ps + 3 * t, pc)) cnt++;
          }
      }
  }
  deg[s] = cnt;
  if (cnt > kMaxRow) atomicOr(flag, 1);
}

// one 64-lane block per row: collect the row's neighbours in LDS, bitonic sort, write
__global__ __launch_bounds__(64) void k_fill(const float* __restrict__ ps, int n, PairCtx pc,
                                              double inv_side, int nc,
                                              const int32_t* __restrict__ cell_start,
                                              const int32_t* __restrict__ cell_atoms,
                                              const int32_t* __restrict__ row_ptr,
                                              int32_t* __restrict__ col) {
  __shared__ int buf[kMaxRow];
  const int s = blockIdx.x;
  const int lane = threadIdx.x;
  const double sx = ps[3 * s], sy = ps[3 * s + 1], sz = ps[3 * s + 2];
  const int expect = row_ptr[s + 1] - row_ptr[s];
  if (expect > kMaxRow) return;
  int count = 0;
  auto consider = [&](int t, bool valid) {
    bool pass = valid && t != s && pair_in(sx, sy, sz, ps + 3 * t, pc);
    uint64_t m = __ballot(pass);
    int pre = __popcll(m & ((1ull << lane) - 1ull));
    if (pass && count + pre < kMaxRow) buf[count + pre] = t;
    count += __popcll(m);
  };
  if (nc == 0) {
    for (int base = 0; base < n; base += 64) {
      int t = base + lane;
      consider(t, t < n);
    }
  } else {
    // The 27 neighbour cells as at most 18 runs of cell_atoms: for each (dx, dy) the cells
    // cz-1, cz, cz+1 are consecutive in the cell order unless they wrap in z (nc >= 3, so
    // no cell is visited twice).  The runs are walked as one list, 64 candidates at a time.
    __shared__ int run_start[18], run_end[19];
    if (lane < 9) {
      const int cx = cell_coord(ps[3 * s], inv_side, nc), cy = cell_coord(ps[3 * s + 1], inv_side, nc),
                cz = cell_coord(ps[3 * s + 2], inv_side, nc);
      int ix = cx + lane / 3 - 1, iy = cy + lane % 3 - 1;
      ix += ix < 0 ? nc : (ix >= nc ? -nc : 0);
      iy += iy < 0 ? nc : (iy >= nc ? -nc : 0);
      const int base = (ix * nc + iy) * nc;
      const int lo = cz > 0 ? cz - 1 : 0, hi = cz + 2 < nc ? cz + 2 : nc;
      run_start[lane] = cell_start[base + lo];
      run_end[lane] = cell_start[base + hi];
      // the wrapped cell, if any: nc - 1 below cz = 0, or 0 above cz = nc - 1 (else empty)
      const int w = cz == 0 ? nc - 1 : (cz == nc - 1 ? 0 : -1);
      run_start[9 + lane] = w >= 0 ? cell_start[base + w] : 0;
      run_end[9 + lane] = w >= 0 ? cell_start[base + w + 1] : 0;
    }
    __syncthreads();
    if (lane == 0) {
      // run_end becomes the exclusive prefix of run lengths (run_end[18] = total)
      int acc = 0;
      for (int r = 0; r < 18; ++r) {
        const int len = run_end[r] - run_start[r];
        run_end[r] = acc;
        acc += len;
      }
      run_end[18] = acc;
    }
    __syncthreads();
    const int total = run_end[18];
    for (int v0 = 0; v0 < total; v0 += 64) {
      const int v = v0 + lane;
      int r = 0;
#pragma unroll
      for (int k = 1; k < 18; ++k) r += v >= run_end[k];
      const bool valid = v < total;
      consider(valid ? cell_atoms[run_start[r] + (v - run_end[r])] : 0, valid);
    }
  }
  __syncthreads();
  int P = 1;
  while (P < count) P <<= 1;
  for (int i = count + lane; i < P; i += 64) buf[i] = INT_MAX;
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = lane; i < P; i += 64) {
        int ixj = i ^ j;
        if (ixj > i) {
          int a = buf[i], b = buf[ixj];
          bool up = (i & k) == 0;
          if ((a > b) == up) {
            buf[i] = b;
            buf[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  const int base = row_ptr[s];
  for (int i = lane; i < count && i < expect; i += 64) col[base + i] = buf[i];
}

// one 64-lane wave per row (4 rows per block), one lane per edge: coalesced col reads
// and rev writes, 64 independent binary searches per wave
constexpr int kRevRows = 4;
__global__ __launch_bounds__(256) void k_rev(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col,
                                             int n, int32_t* __restrict__ rev) {
  const int s = (int)xcd_order(blockIdx.x, gridDim.x, 1024 / kRevRows) * kRevRows + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (s >= n) return;
  for (int e = row_ptr[s] + lane; e < row_ptr[s + 1]; e += 64) {
    int t = col[e];
    int lo = row_ptr[t], hi = row_ptr[t + 1];
    while (lo < hi) {
      int mid = (lo + hi) >> 1;
      if (col[mid] < s) lo = mid + 1;
      else hi = mid;
    }
    rev[e] = lo;
  }
}

// ------------------------------------------------------ batches of open structures
// Many small structures without periodic images, concatenated: structure b holds
// atoms sptr[b] .. sptr[b+1]-1, and an atom's candidates are the other atoms of its
// own structure.  Pair test in float64 with the order of pair_in, no image shifts.
__device__ __forceinline__ bool pair_open(double sx, double sy, double sz, const float* __restrict__ pt, double R2) {
  double d0 = (double)pt[0] - sx;
  double d1 = (double)pt[1] - sy;
  double d2 = (double)pt[2] - sz;
  double a = d0 * d0;
  double b = d1 * d1;
  double c = d2 * d2;
  double D = (a + b) + c;
  return D < R2;
}

// structure index of every atom (a thread per structure; structures are small)
__global__ void k_struct_id(const int32_t* __restrict__ sptr, int nstruct, int32_t* __restrict__ sid) {
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nstruct) return;
  for (int i = sptr[b]; i < sptr[b + 1]; ++i) sid[i] = b;
}

// one 64-lane wave per atom, lanes over the atoms of its structure in ascending
// order: FILL = 0 counts, FILL = 1 writes the row (ascending by construction)
template <int FILL>
__global__ __launch_bounds__(256) void k_open_rows(const float* __restrict__ pos, int n, double R2,
                                                   const int32_t* __restrict__ sptr, const int32_t* __restrict__ sid,
                                                   int32_t* __restrict__ deg, const int32_t* __restrict__ row_ptr,
                                                   int32_t* __restrict__ col) {
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (s >= n) return;
  const int b = sid[s], t0 = sptr[b], t1 = sptr[b + 1];
  const double sx = pos[3 * s], sy = pos[3 * s + 1], sz = pos[3 * s + 2];
  int cnt = 0;
  int out = FILL ? row_ptr[s] : 0;
  for (int base = t0; base < t1; base += 64) {
    const int t = base + lane;
    const bool pass = t < t1 && t != s && pair_open(sx, sy, sz, pos + 3 * t, R2);
    const uint64_t m = __ballot(pass);
    if (FILL && pass) col[out + __popcll(m & ((1ull << lane) - 1ull))] = t;
    out += __popcll(m);
    cnt += __popcll(m);
  }
  if (!FILL && lane == 0) deg[s] = cnt;
}

// fixed-order float64 sum of the atom energies of every structure: one wave per
// structure, lane-strided partial sums, then a butterfly in a fixed order
__global__ __launch_bounds__(256) void k_struct_energy(const float* __restrict__ e_atoms,
                                                       const int32_t* __restrict__ sptr, int nstruct,
                                                       double* __restrict__ out) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (b >= nstruct) return;
  double acc = 0.0;
  for (int i = sptr[b] + lane; i < sptr[b + 1]; i += 64) acc += (double)e_atoms[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) out[b] = acc;
}

}  // namespace nb

// ------------------------------------------------------------- host side
namespace {

struct NbPlan {
  int n, ntiles, nc, ncell, cid_passes;
  int64_t hist_n, scan_blocks;
};

NbPlan plan_nb(int n, float L, float cutoff, float skin) {
  NbPlan p{};
  p.n = n;
  p.ntiles = (int)cdiv(n, nb::kRsTile);
  double R = (double)cutoff + (double)skin;
  int nc = (int)floor((double)L / R);
  // a cell side barely above R invites rounding trouble at cell edges
  while (nc >= 3 && (double)L / nc < R * (1.0 + 1e-6)) nc--;
  p.nc = nc >= 3 ? nc : 0;
  p.ncell = p.nc ? p.nc * p.nc * p.nc : 0;
  int bits = 0;
  while (p.ncell > 0 && (1 << bits) < p.ncell) bits++;
  p.cid_passes = (bits + 7) / 8;
  if (p.cid_passes % 2) p.cid_passes++;  // keep the result in the first buffer
  p.hist_n = 256LL * p.ntiles;
  int64_t m = std::max<int64_t>(std::max<int64_t>(n + 1, p.hist_n), p.ncell + 1);
  p.scan_blocks = cdiv(m, nb::kScBlock);
  return p;
}

struct NbWs {
  float* pos_w;
  uint32_t *k0, *k1;
  int32_t *v0, *v1, *hist, *cell_start, *deg, *flag;
  int64_t *bsum, *total;
};

NbWs carve_nb(Arena& a, const NbPlan& p) {
  NbWs w{};
  w.pos_w = a.take<float>(3LL * p.n);
  w.k0 = a.take<uint32_t>(p.n);
  w.k1 = a.take<uint32_t>(p.n);
  w.v0 = a.take<int32_t>(p.n);
  w.v1 = a.take<int32_t>(p.n);
  w.hist = a.take<int32_t>(p.hist_n + 1);
  w.cell_start = a.take<int32_t>(p.ncell + 1);
  w.deg = a.take<int32_t>(p.n + 1);
  w.flag = a.take<int32_t>(4);
  w.bsum = a.take<int64_t>(p.scan_blocks + 1);
  w.total = a.take<int64_t>(2);
  return w;
}

}  // namespace

// exclusive scan of in[0..n) into out[0..n) (+ out[n] = total if write_total)
int scan_i32(const int32_t* in, int64_t n, int32_t* out, int64_t* bsum, int64_t* total, bool write_total,
             hipStream_t st) {
  int nb_ = (int)cdiv(n, nb::kScBlock);
  if (nb_ < 1) nb_ = 1;
  nb::k_scan_sums<<<nb_, nb::kScThreads, 0, st>>>(in, n, bsum);
  nb::k_scan_partials<<<1, nb::kScThreads, 0, st>>>(bsum, nb_, total);
  nb::k_scan_apply<<<nb_, nb::kScThreads, 0, st>>>(in, n, bsum, out, total, write_total ? 1 : 0);
  MP_CHECK_LAUNCH();
  return MP_OK;
}

static int radix_sort(uint32_t* k0, int32_t* v0, uint32_t* k1, int32_t* v1, int n, int passes,
                      int32_t* hist, int ntiles, int64_t* bsum, int64_t* total, hipStream_t st) {
  for (int ps = 0; ps < passes; ++ps) {
    uint32_t* ki = (ps % 2 == 0) ? k0 : k1;
    int32_t* vi = (ps % 2 == 0) ? v0 : v1;
    uint32_t* ko = (ps % 2 == 0) ? k1 : k0;
    int32_t* vo = (ps % 2 == 0) ? v1 : v0;
    nb::k_radix_hist<<<ntiles, nb::kRsThreads, 0, st>>>(ki, n, 8 * ps, hist, ntiles);
    MP_TRY(scan_i32(hist, 256LL * ntiles, hist, bsum, total, false, st));
    nb::k_radix_scatter<<<ntiles, nb::kRsThreads, 0, st>>>(ki, vi, ko, vo, n, 8 * ps, hist, ntiles);
    MP_CHECK_LAUNCH();
  }
  return MP_OK;
}

}  // namespace mdmp

using namespace mdmp;

extern "C" int mp_build_neighbors_ws(int32_t n, float box_L, float cutoff, float skin, size_t* bytes) {
  if (!bytes || n < 2) return arg_error("mp_build_neighbors_ws: n >= 2 and bytes required");
  NbPlan p = plan_nb(n, box_L, cutoff, skin);
  Arena a(nullptr, 0, true);
  carve_nb(a, p);
  *bytes = a.off;
  return MP_OK;
}

extern "C" int mp_build_neighbors(const float* pos, const int32_t* species, int32_t n, float box_L,
                                  float cutoff, float skin, int32_t* perm, float* pos_sorted,
                                  int32_t* species_sorted, int32_t* row_ptr, int32_t* col, int32_t* rev,
                                  int64_t capacity, int64_t* n_edges, void* ws, size_t ws_bytes,
                                  hipStream_t st) {
  return mp_build_neighbors_ordered(pos, species, n, box_L, cutoff, skin, MP_ORDER_HILBERT, perm, pos_sorted,
                                    species_sorted, row_ptr, col, rev, capacity, n_edges, ws, ws_bytes, st);
}

extern "C" int mp_build_neighbors_ordered(const float* pos, const int32_t* species, int32_t n, float box_L,
                                          float cutoff, float skin, int32_t order, int32_t* perm,
                                          float* pos_sorted, int32_t* species_sorted, int32_t* row_ptr,
                                          int32_t* col, int32_t* rev, int64_t capacity, int64_t* n_edges, void* ws,
                                          size_t ws_bytes, hipStream_t st) {
  if (!pos || !species || !perm || !pos_sorted || !species_sorted || !row_ptr || !n_edges || !ws)
    return arg_error("mp_build_neighbors: null pointer");
  if (order != MP_ORDER_HILBERT && order != MP_ORDER_MORTON && order != MP_ORDER_INPUT)
    return arg_error("mp_build_neighbors: unknown atom order");
  if (n < 2) return arg_error("mp_build_neighbors: n must be >= 2");
  if (!(box_L > 0) || !(cutoff > 0) || !(skin >= 0)) return arg_error("mp_build_neighbors: bad box/cutoff/skin");
  if ((double)cutoff + (double)skin >= 0.5 * (double)box_L) {
    set_error("mp_build_neighbors: r_cut + skin must be < L/2");
    return MP_ERR_BOX;
  }
  NbPlan p = plan_nb(n, box_L, cutoff, skin);
  Arena a(ws, ws_bytes);
  NbWs w = carve_nb(a, p);
  ProfScope prof("build_neighbors", st);
  if (!a.ok()) return arg_error("mp_build_neighbors: workspace too small");

  const int T = 256;
  nb::k_wrap_key<<<cdiv(n, T), T, 0, st>>>(pos, n, box_L, order, w.pos_w, w.k0, w.v0);
  MP_CHECK_LAUNCH();
  MP_TRY(radix_sort(w.k0, w.v0, w.k1, w.v1, n, 4, w.hist, p.ntiles, w.bsum, w.total, st));
  MP_HIP(hipMemcpyAsync(perm, w.v0, sizeof(int32_t) * n, hipMemcpyDeviceToDevice, st));
  nb::k_gather_sorted<<<cdiv(n, T), T, 0, st>>>(perm, w.pos_w, species, n, pos_sorted, species_sorted);
  MP_CHECK_LAUNCH();

  nb::PairCtx pc;
  pc.L = (double)box_L;
  pc.half = 0.5 * pc.L;
  double R = (double)cutoff + (double)skin;
  pc.R2 = R * R;
  double inv_side = p.nc ? (double)p.nc / (double)box_L : 0.0;
  const int32_t* cell_atoms = nullptr;
  if (p.nc) {
    nb::k_cell_id<<<cdiv(n, T), T, 0, st>>>(pos_sorted, n, inv_side, p.nc, w.k0, w.v0);
    MP_CHECK_LAUNCH();
    MP_TRY(radix_sort(w.k0, w.v0, w.k1, w.v1, n, p.cid_passes, w.hist, p.ntiles, w.bsum, w.total, st));
    nb::k_cell_start<<<cdiv(p.ncell + 1, T), T, 0, st>>>(w.k0, n, p.ncell, w.cell_start);
    MP_CHECK_LAUNCH();
    cell_atoms = w.v0;
  }
  MP_HIP(hipMemsetAsync(w.flag, 0, sizeof(int32_t), st));
  nb::k_count<<<cdiv(n, T), T, 0, st>>>(pos_sorted, n, pc, inv_side, p.nc, w.cell_start, cell_atoms,
                                         w.deg, w.flag);
  MP_CHECK_LAUNCH();
  MP_TRY(scan_i32(w.deg, n, row_ptr, w.bsum, w.total, true, st));
  int64_t host[2] = {0, 0};
  MP_HIP(hipMemcpyAsync(&host[0], w.total, sizeof(int64_t), hipMemcpyDeviceToHost, st));
  int32_t hflag = 0;
  MP_HIP(hipMemcpyAsync(&hflag, w.flag, sizeof(int32_t), hipMemcpyDeviceToHost, st));
  MP_HIP(hipStreamSynchronize(st));
  *n_edges = host[0];
  if (hflag) return arg_error("mp_build_neighbors: a row has more than 1024 neighbours");
  if (host[0] > capacity) {
    set_error("mp_build_neighbors: edge capacity too small");
    return MP_ERR_CAPACITY;
  }
  if (host[0] > INT_MAX) return arg_error("mp_build_neighbors: more than 2^31 edges");
  if (!col || !rev) return arg_error("mp_build_neighbors: null col/rev");
  nb::k_fill<<<n, 64, 0, st>>>(pos_sorted, n, pc, inv_side, p.nc, w.cell_start, cell_atoms, row_ptr, col);
  MP_CHECK_LAUNCH();
  nb::k_rev<<<cdiv(n, nb::kRevRows), 256, 0, st>>>(row_ptr, col, n, rev);
  MP_CHECK_LAUNCH();
  return MP_OK;
}

extern "C" int mp_build_neighbors_batched_ws(int32_t n, int32_t n_struct, size_t* bytes) {
  if (!bytes || n < 1 || n_struct < 1) return arg_error("mp_build_neighbors_batched_ws: n, n_struct >= 1 and bytes required");
  Arena a(nullptr, 0, true);
  a.take<int32_t>(n + 1);                                 // structure id per atom
  a.take<int32_t>(n + 1);                                 // degrees
  a.take<int64_t>(cdiv((int64_t)n + 1, nb::kScBlock) + 1);  // scan block sums
  a.take<int64_t>(2);                                     // total
  *bytes = a.off;
  return MP_OK;
}

extern "C" int mp_build_neighbors_batched(const float* pos, int32_t n, const int32_t* struct_ptr, int32_t n_struct,
                                          float cutoff, float skin, int32_t* row_ptr, int32_t* col, int32_t* rev,
                                          int64_t capacity, int64_t* n_edges, void* ws, size_t ws_bytes,
                                          hipStream_t st) {
  if (!pos || !struct_ptr || !row_ptr || !n_edges || !ws) return arg_error("mp_build_neighbors_batched: null pointer");
  if (n < 1 || n_struct < 1) return arg_error("mp_build_neighbors_batched: n, n_struct >= 1 required");
  if (!(cutoff > 0) || !(skin >= 0)) return arg_error("mp_build_neighbors_batched: bad cutoff/skin");
  Arena a(ws, ws_bytes);
  int32_t* sid = a.take<int32_t>(n + 1);
  int32_t* deg = a.take<int32_t>(n + 1);
  int64_t* bsum = a.take<int64_t>(cdiv((int64_t)n + 1, nb::kScBlock) + 1);
  int64_t* total = a.take<int64_t>(2);
  if (!a.ok()) return arg_error("mp_build_neighbors_batched: workspace too small");
  ProfScope prof("build_neighbors", st);
  const double R = (double)cutoff + (double)skin;
  const int T = 256;
  nb::k_struct_id<<<cdiv(n_struct, T), T, 0, st>>>(struct_ptr, n_struct, sid);
  MP_CHECK_LAUNCH();
  nb::k_open_rows<0><<<cdiv(n, 4), T, 0, st>>>(pos, n, R * R, struct_ptr, sid, deg, nullptr, nullptr);
  MP_CHECK_LAUNCH();
  MP_TRY(scan_i32(deg, n, row_ptr, bsum, total, true, st));
  int64_t host = 0;
  MP_HIP(hipMemcpyAsync(&host, total, sizeof(int64_t), hipMemcpyDeviceToHost, st));
  MP_HIP(hipStreamSynchronize(st));
  *n_edges = host;
  if (host > capacity) {
    set_error("mp_build_neighbors_batched: edge capacity too small");
    return MP_ERR_CAPACITY;
  }
  if (host > INT_MAX) return arg_error("mp_build_neighbors_batched: more than 2^31 edges");
  if (host == 0) return MP_OK;
  if (!col || !rev) return arg_error("mp_build_neighbors_batched: null col/rev");
  nb::k_open_rows<1><<<cdiv(n, 4), T, 0, st>>>(pos, n, R * R, struct_ptr, sid, nullptr, row_ptr, col);
  MP_CHECK_LAUNCH();
  nb::k_rev<<<cdiv(n, nb::kRevRows), 256, 0, st>>>(row_ptr, col, n, rev);
  MP_CHECK_LAUNCH();
  return MP_OK;
}

extern "C" int mp_structure_energies(const float* atom_energy, const int32_t* struct_ptr, int32_t n_struct,
                                     double* energies, hipStream_t st) {
  if (!atom_energy || !struct_ptr || !energies || n_struct < 1) return arg_error("mp_structure_energies: bad arguments");
  nb::k_struct_energy<<<cdiv(n_struct, 4), 256, 0, st>>>(atom_energy, struct_ptr, n_struct, energies);
  MP_CHECK_LAUNCH();
  return MP_OK;
}

