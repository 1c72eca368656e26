// Host-visible structures shared by the model kernels and the C ABI.
#pragma once
#include "common.hpp"

struct mp_model;
struct mp_heads;

namespace mdmp {

struct LayerW {
  const float* w1;       // [64][8]
  const float* w2;       // [P*C][64]
  const uint16_t* w2b;   // bf16 copy of w2
  const float* w2t;      // [64][P*C] transposed
  const uint16_t* w2tb;  // bf16 copy of w2t
  // bf16 W_2 and W_2^T in the order the edge kernels' waves read their MFMA fragments,
  // one copy per path set (index = layer mode 0, 1, 2: all paths, l1 = 0, l3 = 0) over
  // that mode's channel blocks of CB (32 unpruned, 64 pruned; null below 32 channels):
  // each 64-lane fragment load reads 1 KB of consecutive bytes
  const uint16_t* w2sw[3];   // [C/CB][NA*CB/16][2][64][8]: 16-row block, half, lane, unit
  const uint16_t* w2tsw[3];  // [C/CB][4][NA*CB/32][64][8]: hidden block, 32-wide k step, lane, unit
  // the float32 kernels' fragment order (channel blocks of 32 in every mode): W_2 as
  // [C/32][NA*2][4][64][4] (16-row block, 4-unit step, lane, unit) and W_2^T as
  // [C/32][4][NA*2][64][4] (hidden block, 4-wide k step of each lane group, lane, unit)
  const float* w2sf[3];
  const float* w2tsf[3];
  const float* wq;       // [C][C]  (out, in)
  const float* wqT;      // [C][C]  (in, out)
  const float* wv[3];
  const float* wvT[3];
  const float* wo[3];
  const float* woT[3];
  const float* wg;       // [L*C][C]
  const float* wgT;      // [C][L*C]
  // (wq .. wgT above and the bf16 copies below are in the per-atom kernels' MFMA
  // fragment order, [rows/16][cols/CK][64][EV]; see load_a)
  // bf16 copies for the MFMA per-atom products (bf16 feature configurations)
  const uint16_t *wq_b, *wqT_b, *wg_b, *wgT_b;
  const uint16_t* wv_b[3];
  const uint16_t* wvT_b[3];
  const uint16_t* wo_b[3];
  const uint16_t* woT_b[3];
};

// The narrowest channel block of the edge kernels (32; C itself below 32): the
// per-edge geometry gradients are kept in one slab per such block.
constexpr int edge_channel_block(int C, bool) { return C < 32 ? C : 32; }

struct Plan {
  int n, lmax, C, H, T, K, NP;
  bool bf16;
  int64_t cap;  // padded edge capacity
  int ncb;      // channel blocks
};

// floats per active-edge geometry record in HBM (r, u, du/dr, rhat[3], B[8], 0, 0)
constexpr int kGeoFloats = 16;

// Active edges (r < r_cut) of row i at row_ptr[i] .. aend[i] - 1 of the padded edge
// arrays (compacted in order at the front of the row's padded range).
// slots per half of the geometry-gradient partials: ceil(ncb / 2)
inline int gd_half_slots(const Plan& P) { return (P.ncb + 1) / 2; }
// floats of the geometry-gradient partials: two halves of [cap][half slots][3]
inline int64_t gd_floats(const Plan& P) { return 2 * (int64_t)gd_half_slots(P) * P.cap * 3; }

struct Geo {
  int32_t *aend, *a_j, *a_r, *amap, *arev;  // a_r: padded index of the reverse edge
  float* geo;  // [cap][kGeoH]
};

struct EdgeArgs {
  const int32_t* abeg;  // the graph's row_ptr
  const int32_t* aend;
  const int32_t* a_j;
  const int32_t* arev;
  const float* geo;
  const void* ht;
  const float* q;
  float* mz;  // [n][H][2] (max, normaliser)
  int dh, heads;
  float rc;
};

struct BwdArgs {
  const void* m_saved;
  float* g_m;
  float* g_ht;
  float* g_q;
  float* ag;   // [cap][H][2] (alpha, dE/dlogit)
  // per-edge partials of dE/dd, one per slot of edge_channel_block() channels: slot s in
  // half s % 2 at [cap][gd_half][3] (index s / 2), added up by the force gather
  float* gd;
  int64_t gd_cap;
  int gd_half;  // gd_half_slots(plan)
};

int scan_i32(const int32_t* in, int64_t n, int32_t* out, int64_t* bsum, int64_t* total, bool write_total,
             hipStream_t st);
int geometry(const Plan& P, const mp_graph* g, float rc, Geo& G, hipStream_t st);
// mode: bit 1 = first layer (only l1 = 0 paths), bit 2 = last layer of an energy
// evaluation (only l3 = 0 paths); 0 = the full layer
int dispatch_layer_fwd(const Plan& P, const EdgeArgs& A, const LayerW& W, const void* h_in, void* h_out, void* ht,
                       float* q, void* m, int mode, hipStream_t st);
// zero_rows: also write the feature rows l > 0 (zeros); an energy evaluation, whose first
// layer reads only row 0, leaves them out
int dispatch_embed(const Plan& P, const float* emb, const int32_t* sp, void* h, bool zero_rows, hipStream_t st);
// R readout heads on the same features: head k's [C][C] matrices at wrT / wr + k C^2,
// its output weights at wout + k C; e_atoms [R][n].  lam (device [R], nullable = all 1)
// weights each head's gradient.  R = 1 with the model's weights is the model's readout.
int dispatch_readout(const Plan& P, int R, const void* h, const float* wrT, const float* wout, float* e_atoms,
                     hipStream_t st);
int dispatch_readout_bwd(const Plan& P, int R, const void* h, const float* wrT, const float* wr, const float* wout,
                         const float* lam, float* g_h, hipStream_t st);
// input_grad: also form the gradient with respect to the layer's input features (not
// needed for the first layer, whose input does not depend on positions)
int dispatch_layer_bwd(const Plan& P, const EdgeArgs& A, const LayerW& W, const BwdArgs& B, float* g_h, int mode,
                       bool input_grad, hipStream_t st);
// F_k = sum over row k's active edges a of (dE/dd_a - dE/dd_{arev[a]}), each dE/dd the
// sum of its channel-block partials in gd
int launch_forces(const Plan& P, const mp_graph* g, const Geo& G, const float* gd, const int32_t* perm, float* F,
                  int32_t* flag, hipStream_t st);
int launch_energy(const float* e_atoms, int n, double* out, int32_t* flag, hipStream_t st);
// *out = sum_k lam_k e[k] over k = 0..R-1 in float64, in index order; flag set if not finite
int launch_weighted_sum(const double* e, const float* lam, int R, double* out, int32_t* flag, hipStream_t st);
bool supported(int lmax, int C, bool bf16);
int fill_zero(void* p, size_t bytes, hipStream_t st);
// heads (nullable): readout heads replacing the model's own; then atom_energy is the
// [R][n] per-head atom energies, head_energy [R] the heads' energies and energy their
// lam-weighted sum, whose gradient the reverse pass follows
int ef_enqueue(const mp_model* m, const mp_graph* g, int64_t cap, const int32_t* perm, double* energy, float* forces,
               float* atom_energy, void* ws, size_t ws_bytes, int32_t** flag_out, hipStream_t st,
               const mp_heads* heads = nullptr, double* head_energy = nullptr);

}  // namespace mdmp

struct mp_heads {
  int32_t R = 0, C = 0;
  float* dev = nullptr;  // one allocation for the arrays below
  const float *wr, *wrT, *wout, *lam;
};

struct mp_model {
  mp_model_config cfg;
  mdmp::Plan base;        // n and cap unset
  void* dev = nullptr;    // one allocation for every weight array
  mdmp::LayerW layers[16];
  const float *emb, *wr, *wrT, *wout;
};
