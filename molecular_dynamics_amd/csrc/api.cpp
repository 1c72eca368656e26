// C ABI of libmdmp: model handles, workspace planning, energy + forces.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

#include "cg_real.hpp"
#include "model.hpp"

namespace mdmp {

static thread_local std::string g_err;
void set_error(const std::string& msg) { g_err = msg; }

static uint16_t host_f2bf(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static int n_paths(int lmax) {
  int n = 0;
  for (int a = 0; a <= lmax; ++a)
    for (int b = 0; b <= lmax; ++b)
      for (int c = 0; c <= lmax; ++c)
        if (c >= std::abs(a - b) && c <= a + b) n++;
  return n;
}

static int64_t count_weights(const mp_model_config& c) {
  const int64_t C = c.channels, P = n_paths(c.lmax);
  int64_t per = 64 * 8 + P * C * 64 + C * C + 2 * (c.lmax + 1) * C * C + c.lmax * C * C;
  return c.n_species * C + c.layers * per + C * C + C;
}

static int validate(const mp_model_config* c) {
  if (!c) return arg_error("null config");
  if (c->lmax != 1 && c->lmax != 2) return arg_error("lmax must be 1 or 2");
  if (c->n_bessel != 8 || c->radial_hidden != 64) return arg_error("n_bessel must be 8 and radial_hidden 64");
  if (c->heads < 1 || c->channels % c->heads) return arg_error("heads must divide channels");
  int dh = c->channels / c->heads;
  if (dh & (dh - 1)) return arg_error("channels per head must be a power of two");
  // a head's logit is summed inside one channel block of the edge kernels
  if (dh > edge_channel_block(c->channels, c->feat_dtype == 1))
    return arg_error("a head may span at most 32 channels");
  if (c->layers < 1 || c->layers > 16) return arg_error("layers must be in 1..16");
  if (c->n_species < 1) return arg_error("n_species must be >= 1");
  if (!(c->cutoff > 0)) return arg_error("cutoff must be > 0");
  if (c->feat_dtype != 0 && c->feat_dtype != 1) return arg_error("feat_dtype must be 0 or 1");
  if (!supported(c->lmax, c->channels, c->feat_dtype == 1))
    return arg_error("unsupported (lmax, channels, feat_dtype); built: (1,16,f32) (2,16,f32) (2,64,*) "
                     "(2,128,*) (1,64,f32)");
  return MP_OK;
}

// --------------------------------------------------------------- workspace
struct EfWs {
  Geo G;
  void* h;                    // current features
  void *ht, *m;               // [T] saved
  float *q, *mz;              // [T] saved
  float *g_h, *g_m, *g_ht, *g_q, *ag, *gd, *e_atoms;
  int32_t* flag;
};

static size_t feat_bytes(const Plan& P) { return (size_t)P.n * P.K * P.C * (P.bf16 ? 2 : 4); }

static void carve_geo(Arena& a, const Plan& P, Geo& G) {
  G.aend = a.take<int32_t>(P.n);
  G.a_j = a.take<int32_t>(P.cap);
  G.a_r = a.take<int32_t>(P.cap);
  G.amap = a.take<int32_t>(P.cap);
  G.arev = a.take<int32_t>(P.cap);
  G.geo = a.take<float>(P.cap * kGeoFloats);
}

static EfWs carve_ef(Arena& a, const Plan& P, bool backward) {
  EfWs w{};
  w.flag = a.take<int32_t>(4);  // first: mp_energy_forces_status reads it at offset 0
  carve_geo(a, P, w.G);
  const size_t fb = feat_bytes(P);
  w.h = a.take<char>(fb);
  w.ht = a.take<char>(fb * P.T);
  w.m = a.take<char>(fb * P.T);
  w.q = a.take<float>((int64_t)P.T * P.n * P.C);
  w.mz = a.take<float>((int64_t)P.T * P.n * P.H * 2);
  w.e_atoms = a.take<float>(P.n);
  if (backward) {
    const int64_t nf = (int64_t)P.n * P.K * P.C;
    w.g_h = a.take<float>(nf);
    w.g_m = a.take<float>(nf);
    w.g_ht = a.take<float>(nf);
    w.g_q = a.take<float>((int64_t)P.n * P.C);
    w.ag = a.take<float>(P.cap * P.H * 2);
    w.gd = a.take<float>(gd_floats(P));
  }
  return w;
}

static Plan make_plan(const mp_model* m, int32_t n, int64_t cap) {
  Plan P = m->base;
  P.n = n;
  P.cap = cap > 0 ? cap : 1;
  return P;
}

static EdgeArgs edge_args(const mp_model* m, const Plan& P, const mp_graph* g, const Geo& G) {
  EdgeArgs A{};
  A.abeg = g->row_ptr;
  A.aend = G.aend;
  A.a_j = G.a_j;
  A.arev = G.arev;
  A.geo = G.geo;
  A.dh = P.C / P.H;
  A.heads = P.H;
  A.rc = m->cfg.cutoff;
  return A;
}

static int check_graph(const mp_model* m, const mp_graph* g) {
  if (!m || !g) return arg_error("null model or graph");
  if (g->n < 1 || !g->pos || !g->species || !g->row_ptr) return arg_error("graph: bad n or null arrays");
  if (g->n_edges > 0 && (!g->col || !g->rev)) return arg_error("graph: null col/rev");
  if (!(g->box_L >= 0) || !std::isfinite(g->box_L)) return arg_error("graph: box_L must be >= 0 (0: open boundary)");
  if (g->box_L > 0 && (double)m->cfg.cutoff >= 0.5 * (double)g->box_L) {
    set_error("cutoff must be < L/2");
    return MP_ERR_BOX;
  }
  return MP_OK;
}

}  // namespace mdmp

using namespace mdmp;

extern "C" int mp_version(void) { return 1; }
extern "C" const char* mp_last_error(void) { return g_err.c_str(); }

extern "C" int mp_model_num_weights(const mp_model_config* cfg, int64_t* n) {
  MP_TRY(validate(cfg));
  if (!n) return arg_error("null n");
  *n = count_weights(*cfg);
  return MP_OK;
}

extern "C" int mp_cg_table(int32_t lmax, double* out, int64_t cap, int64_t* n_rows) {
  if (lmax != 1 && lmax != 2) return arg_error("lmax must be 1 or 2");
  if (!n_rows) return arg_error("null n_rows");
  const cgc::Table& T = lmax == 1 ? cgc::kTable1 : cgc::kTable2;
  int64_t r = 0;
  for (int p = 0; p < T.npaths; ++p)
    for (int z = 0; z < T.p[p].nnz; ++z, ++r) {
      if (!out || r >= cap) continue;
      double* o = out + 7 * r;
      o[0] = T.p[p].l1;
      o[1] = T.p[p].l2;
      o[2] = T.p[p].l3;
      o[3] = T.p[p].m1[z];
      o[4] = T.p[p].m2[z];
      o[5] = T.p[p].m3[z];
      o[6] = T.p[p].v[z];
    }
  *n_rows = r;
  return MP_OK;
}

extern "C" int mp_model_create(const mp_model_config* cfg, const float* w, int64_t nw, mp_model** out) {
  MP_TRY(validate(cfg));
  if (!w || !out) return arg_error("null weights or out");
  if (nw != count_weights(*cfg)) return arg_error("weight count does not match the configuration");
  const int C = cfg->channels, L = cfg->lmax, P = n_paths(L), T = cfg->layers;
  // host staging: [original fp32 blob][transposes][bf16 W_2 copies]
  std::vector<float> tr;  // transposed matrices, appended in a fixed order
  std::vector<uint16_t> w2b;
  std::vector<float> swf;  // float32 per-atom matrices in fragment order
  auto transpose = [&](const float* src, int rows, int cols) {
    size_t off = tr.size();
    tr.resize(off + (size_t)rows * cols);
    for (int r = 0; r < rows; ++r)
      for (int c2 = 0; c2 < cols; ++c2) tr[off + (size_t)c2 * rows + r] = src[(size_t)r * cols + c2];
    return off;
  };
  struct Offs {
    size_t w1, w2, wq, wv[3], wo[3], wg, wqT, wvT[3], woT[3], wgT, w2b, w2t, w2tb, w2sw[3], w2tsw[3], w2sf[3],
        w2tsf[3];
    size_t wq_b, wqT_b, wg_b, wgT_b, wv_b[3], wvT_b[3], wo_b[3], woT_b[3];
    size_t wq_s, wqT_s, wg_s, wgT_s, wv_s[3], wvT_s[3], wo_s[3], woT_s[3];  // float32, fragment order
  };
  std::vector<Offs> lo(T);
  size_t p = 0;
  const size_t emb = p;
  p += (size_t)cfg->n_species * C;
  for (int t = 0; t < T; ++t) {
    Offs& o = lo[t];
    o.w1 = p;
    p += 64 * 8;
    o.w2 = p;
    p += (size_t)P * C * 64;
    o.wq = p;
    p += (size_t)C * C;
    for (int l = 0; l <= L; ++l) {
      o.wv[l] = p;
      p += (size_t)C * C;
    }
    for (int l = 0; l <= L; ++l) {
      o.wo[l] = p;
      p += (size_t)C * C;
    }
    o.wg = p;
    p += (size_t)L * C * C;
  }
  const size_t wr = p;
  p += (size_t)C * C;
  const size_t wout = p;
  p += C;
  if ((int64_t)p != nw) return arg_error("internal: weight layout mismatch");
  for (int t = 0; t < T; ++t) {
    Offs& o = lo[t];
    o.wqT = transpose(w + o.wq, C, C);
    for (int l = 0; l <= L; ++l) o.wvT[l] = transpose(w + o.wv[l], C, C);
    for (int l = 0; l <= L; ++l) o.woT[l] = transpose(w + o.wo[l], C, C);
    o.wgT = transpose(w + o.wg, L * C, C);
    o.w2b = w2b.size();
    for (size_t q = 0; q < (size_t)P * C * 64; ++q) w2b.push_back(host_f2bf(w[o.w2 + q]));
    o.w2t = transpose(w + o.w2, P * C, 64);
    o.w2tb = w2b.size();
    for (size_t q = 0; q < (size_t)P * C * 64; ++q) w2b.push_back(host_f2bf(tr[o.w2t + q]));
    // the same two matrices in the edge kernels' fragment order, one copy per path set
    // (mode 0: all paths, channel blocks of 32; modes 1 and 2: the paths with l1 = 0 or
    // l3 = 0, channel blocks of min(C, 64)).  W_2: lane l = 16 g + e of the fragment of
    // 16-row block rb holds row (path q, channel CB cb + (16 rb) mod CB + e), q = 16 rb / CB,
    // hidden units 16 g + 8 half .. + 7.  W_2^T: lane l of hidden block hb, k step t holds
    // hidden unit 16 hb + (l mod 16), entries k = 32 t + 8 (l / 16) .. + 7 of (path q =
    // k / CB, channel CB cb + k mod CB).
    for (int mode = 0; mode < 3; ++mode) {
      o.w2sw[mode] = o.w2tsw[mode] = o.w2sf[mode] = o.w2tsf[mode] = 0;
      if (C < 32) continue;
      std::vector<int> pl;
      const cgc::Table& tab = L == 1 ? cgc::TableOf<1>::t : cgc::TableOf<2>::t;
      for (int pp = 0; pp < tab.npaths; ++pp)
        if (!((mode & 1) && tab.p[pp].l1 != 0) && !((mode & 2) && tab.p[pp].l3 != 0)) pl.push_back(pp);
      const int NA = (int)pl.size(), CB = mode == 0 ? 32 : std::min(C, 64);
      o.w2sw[mode] = w2b.size();
      for (int cb = 0; cb < C / CB; ++cb)
        for (int rb = 0; rb < NA * CB / 16; ++rb)
          for (int half = 0; half < 2; ++half)
            for (int l = 0; l < 64; ++l)
              for (int j2 = 0; j2 < 8; ++j2) {
                const size_t row = (size_t)pl[rb * 16 / CB] * C + CB * cb + (16 * rb) % CB + (l & 15);
                w2b.push_back(host_f2bf(w[o.w2 + row * 64 + 16 * (l >> 4) + 8 * half + j2]));
              }
      o.w2tsw[mode] = w2b.size();
      for (int cb = 0; cb < C / CB; ++cb)
        for (int hb = 0; hb < 4; ++hb)
          for (int t2 = 0; t2 < NA * CB / 32; ++t2)
            for (int l = 0; l < 64; ++l)
              for (int j2 = 0; j2 < 8; ++j2) {
                const size_t h = 16 * hb + (l & 15);
                const int k = 32 * t2 + 8 * (l >> 4) + j2;
                w2b.push_back(host_f2bf(tr[o.w2t + h * ((size_t)P * C) + (size_t)pl[k / CB] * C + CB * cb + k % CB]));
              }
      // float32 kernels (channel blocks of 32 in every mode): W_2 lane l = 16 g + e of
      // 16-row block rb, step i holds hidden units 16 g + 4 i .. + 3 of its row; W_2^T lane l
      // of hidden block hb, step s holds k = (l / 16) KT/4 + 4 s .. + 3, KT = 32 NA
      const int CF = 32, KT = NA * CF;
      o.w2sf[mode] = tr.size();
      for (int cb = 0; cb < C / CF; ++cb)
        for (int rb = 0; rb < NA * CF / 16; ++rb)
          for (int i4 = 0; i4 < 4; ++i4)
            for (int l = 0; l < 64; ++l)
              for (int z = 0; z < 4; ++z) {
                const size_t row = (size_t)pl[rb * 16 / CF] * C + CF * cb + (16 * rb) % CF + (l & 15);
                tr.push_back(w[o.w2 + row * 64 + 16 * (l >> 4) + 4 * i4 + z]);
              }
      o.w2tsf[mode] = tr.size();
      for (int cb = 0; cb < C / CF; ++cb)
        for (int hb = 0; hb < 4; ++hb)
          for (int st = 0; st < KT / 16; ++st)
            for (int l = 0; l < 64; ++l)
              for (int z = 0; z < 4; ++z) {
                const size_t h = 16 * hb + (l & 15);
                const int k = (l >> 4) * (KT / 4) + 4 * st + z;
                const float v = tr[o.w2t + h * ((size_t)P * C) + (size_t)pl[k / CF] * C + CF * cb + k % CF];
                tr.push_back(v);  // a copy first: push_back may reallocate tr
              }
    }
    // every per-atom matrix and its transpose in the per-atom kernels' MFMA fragment
    // order, [R/16][cols/CK][64 lanes][EPL]: lane l of the fragment of row tile rt and
    // column chunk cc holds row 16 rt + l mod 16, columns CK cc + EPL (l / 16) .. + EPL - 1
    // (bf16: CK 32, EPL 8; float32: CK 16, EPL 4), so each 64-lane load reads 1 KB of
    // consecutive bytes
    auto swz_b = [&](const float* src, int R, int cols) {
      size_t off = w2b.size();
      for (int rt = 0; rt < R / 16; ++rt)
        for (int cc = 0; cc < cols / 32; ++cc)
          for (int l = 0; l < 64; ++l)
            for (int j2 = 0; j2 < 8; ++j2)
              w2b.push_back(host_f2bf(src[(size_t)(16 * rt + (l & 15)) * cols + 32 * cc + 8 * (l >> 4) + j2]));
      return off;
    };
    auto swz_f = [&](const float* src, int R, int cols) {
      size_t off = swf.size();
      for (int rt = 0; rt < R / 16; ++rt)
        for (int cc = 0; cc < cols / 16; ++cc)
          for (int l = 0; l < 64; ++l)
            for (int z = 0; z < 4; ++z) swf.push_back(src[(size_t)(16 * rt + (l & 15)) * cols + 16 * cc + 4 * (l >> 4) + z]);
      return off;
    };
    o.wq_b = swz_b(w + o.wq, C, C);
    o.wqT_b = swz_b(tr.data() + o.wqT, C, C);
    o.wg_b = swz_b(w + o.wg, L * C, C);
    o.wgT_b = swz_b(tr.data() + o.wgT, C, L * C);
    o.wq_s = swz_f(w + o.wq, C, C);
    o.wqT_s = swz_f(tr.data() + o.wqT, C, C);
    o.wg_s = swz_f(w + o.wg, L * C, C);
    o.wgT_s = swz_f(tr.data() + o.wgT, C, L * C);
    for (int l = 0; l <= L; ++l) {
      o.wv_b[l] = swz_b(w + o.wv[l], C, C);
      o.wvT_b[l] = swz_b(tr.data() + o.wvT[l], C, C);
      o.wo_b[l] = swz_b(w + o.wo[l], C, C);
      o.woT_b[l] = swz_b(tr.data() + o.woT[l], C, C);
      o.wv_s[l] = swz_f(w + o.wv[l], C, C);
      o.wvT_s[l] = swz_f(tr.data() + o.wvT[l], C, C);
      o.wo_s[l] = swz_f(w + o.wo[l], C, C);
      o.woT_s[l] = swz_f(tr.data() + o.woT[l], C, C);
    }
  }
  const size_t wrT = transpose(w + wr, C, C);
  const size_t b_main = align_up(sizeof(float) * nw), b_tr = align_up(sizeof(float) * tr.size());
  const size_t b_bf = align_up(sizeof(uint16_t) * (w2b.size() + 8));
  const size_t b_sw = align_up(sizeof(float) * (swf.size() + 4));
  mp_model* m = new mp_model();
  m->cfg = *cfg;
  char* dev = nullptr;
  hipError_t e = hipMalloc((void**)&dev, b_main + b_tr + b_bf + b_sw);
  if (e != hipSuccess) {
    delete m;
    set_error(std::string("hipMalloc: ") + hipGetErrorString(e));
    return MP_ERR_HIP;
  }
  m->dev = dev;
  float* dw = (float*)dev;
  float* dt = (float*)(dev + b_main);
  uint16_t* db = (uint16_t*)(dev + b_main + b_tr);
  float* ds = (float*)(dev + b_main + b_tr + b_bf);
  if (hipMemcpy(dw, w, sizeof(float) * nw, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(dt, tr.data(), sizeof(float) * tr.size(), hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(db, w2b.data(), sizeof(uint16_t) * w2b.size(), hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(ds, swf.data(), sizeof(float) * swf.size(), hipMemcpyHostToDevice) != hipSuccess) {
    hipFree(dev);
    delete m;
    set_error("hipMemcpy of weights failed");
    return MP_ERR_HIP;
  }
  for (int t = 0; t < T; ++t) {
    Offs& o = lo[t];
    LayerW& W = m->layers[t];
    W = LayerW{};
    W.w1 = dw + o.w1;
    W.w2 = dw + o.w2;
    W.w2b = db + o.w2b;
    W.w2t = dt + o.w2t;
    W.w2tb = db + o.w2tb;
    for (int mode = 0; mode < 3; ++mode) {
      W.w2sw[mode] = C >= 32 ? db + o.w2sw[mode] : nullptr;
      W.w2tsw[mode] = C >= 32 ? db + o.w2tsw[mode] : nullptr;
      W.w2sf[mode] = C >= 32 ? dt + o.w2sf[mode] : nullptr;
      W.w2tsf[mode] = C >= 32 ? dt + o.w2tsf[mode] : nullptr;
    }
    W.wq_b = db + o.wq_b;
    W.wqT_b = db + o.wqT_b;
    W.wg_b = db + o.wg_b;
    W.wgT_b = db + o.wgT_b;
    for (int l = 0; l <= L; ++l) {
      W.wv_b[l] = db + o.wv_b[l];
      W.wvT_b[l] = db + o.wvT_b[l];
      W.wo_b[l] = db + o.wo_b[l];
      W.woT_b[l] = db + o.woT_b[l];
    }
    // the per-atom products read these through their fragment-ordered copies
    W.wq = ds + o.wq_s;
    W.wqT = ds + o.wqT_s;
    for (int l = 0; l <= L; ++l) {
      W.wv[l] = ds + o.wv_s[l];
      W.wvT[l] = ds + o.wvT_s[l];
      W.wo[l] = ds + o.wo_s[l];
      W.woT[l] = ds + o.woT_s[l];
    }
    W.wg = ds + o.wg_s;
    W.wgT = ds + o.wgT_s;
  }
  m->emb = dw + emb;
  m->wr = dw + wr;
  m->wrT = dt + wrT;
  m->wout = dw + wout;
  Plan& B = m->base;
  B = Plan{};
  B.lmax = L;
  B.C = C;
  B.H = cfg->heads;
  B.T = T;
  B.K = (L + 1) * (L + 1);
  B.NP = P;
  B.bf16 = cfg->feat_dtype == 1;
  B.ncb = C / edge_channel_block(C, B.bf16);
  *out = m;
  return MP_OK;
}

extern "C" int mp_model_destroy(mp_model* m) {
  if (!m) return MP_OK;
  if (m->dev) hipFree(m->dev);
  delete m;
  return MP_OK;
}

extern "C" int mp_energy_forces_ws(const mp_model* m, int32_t n, int64_t n_edges, size_t* bytes) {
  if (!m || !bytes || n < 1 || n_edges < 0) return arg_error("mp_energy_forces_ws: bad arguments");
  Plan P = make_plan(m, n, n_edges);
  Arena a(nullptr, 0, true);
  carve_ef(a, P, true);
  *bytes = a.off;
  return MP_OK;
}

extern "C" int mp_layer_forward_ws(const mp_model* m, int32_t n, int64_t n_edges, size_t* bytes) {
  if (!m || !bytes || n < 1 || n_edges < 0) return arg_error("mp_layer_forward_ws: bad arguments");
  Plan P = make_plan(m, n, n_edges);
  P.T = 1;
  Arena a(nullptr, 0, true);
  carve_ef(a, P, false);
  *bytes = a.off;
  return MP_OK;
}

extern "C" int mp_embed(const mp_model* m, const mp_graph* g, void* h_out, hipStream_t st) {
  MP_TRY(check_graph(m, g));
  if (!h_out) return arg_error("null h_out");
  if ((uintptr_t)h_out & 15) return arg_error("h_out must be 16-byte aligned");
  Plan P = make_plan(m, g->n, g->n_edges);
  return dispatch_embed(P, m->emb, g->species, h_out, true, st);
}

extern "C" int mp_layer_forward(const mp_model* m, int32_t layer, const mp_graph* g, const void* h_in, void* h_out,
                                void* ws, size_t ws_bytes, hipStream_t st) {
  MP_TRY(check_graph(m, g));
  if (layer < 0 || layer >= m->cfg.layers) return arg_error("layer out of range");
  if (!h_in || !h_out || !ws) return arg_error("null h_in/h_out/ws");
  if (((uintptr_t)h_in | (uintptr_t)h_out) & 15) return arg_error("h_in and h_out must be 16-byte aligned");
  Plan P = make_plan(m, g->n, g->n_edges);
  P.T = 1;
  Arena a(ws, ws_bytes);
  EfWs w = carve_ef(a, P, false);
  if (!a.ok()) return arg_error("mp_layer_forward: workspace too small");
  MP_TRY(geometry(P, g, m->cfg.cutoff, w.G, st));
  EdgeArgs A = edge_args(m, P, g, w.G);
  A.mz = w.mz;
  return dispatch_layer_fwd(P, A, m->layers[layer], h_in, h_out, w.ht, w.q, w.m, 0, st);
}

namespace mdmp {
// Inside an energy evaluation the first layer sees h^{l>0} = 0 exactly, so only
// paths with l1 = 0 contribute; after the last layer only h^0 reaches the
// readout, so only paths with l3 = 0 matter.  Both restrictions are exact.
static int layer_mode(int t, int T) { return (t == 0 ? 1 : 0) | (t == T - 1 ? 2 : 0); }

// Enqueue the whole energy + force evaluation; no host synchronisation and no
// memset nodes, so the sequence can be captured into a hipGraph.  cap is the
// edge capacity the workspace was planned for.  flag (device int) collects
// non-finite outputs.
int ef_enqueue(const mp_model* m, const mp_graph* g, int64_t cap, const int32_t* perm, double* energy, float* forces,
               float* atom_energy, void* ws, size_t ws_bytes, int32_t** flag_out, hipStream_t st,
               const mp_heads* heads, double* head_energy) {
  MP_TRY(check_graph(m, g));
  if (!energy || !forces || !ws) return arg_error("null energy/forces/ws");
  if (g->n_edges > cap) return arg_error("graph has more edges than the workspace capacity");
  Plan P = make_plan(m, g->n, cap);
  Arena a(ws, ws_bytes);
  EfWs w = carve_ef(a, P, true);
  if (!a.ok()) return arg_error("mp_energy_forces: workspace too small");
  const size_t fb = feat_bytes(P);
  MP_TRY(geometry(P, g, m->cfg.cutoff, w.G, st));
  EdgeArgs A = edge_args(m, P, g, w.G);
  // the first layer reads only the scalar rows of its input (layer_mode bit 1)
  MP_TRY(dispatch_embed(P, m->emb, g->species, w.h, false, st));
  for (int t = 0; t < P.T; ++t) {
    A.mz = w.mz + (size_t)t * P.n * P.H * 2;
    MP_TRY(dispatch_layer_fwd(P, A, m->layers[t], w.h, w.h, (char*)w.ht + fb * t, w.q + (size_t)t * P.n * P.C,
                              (char*)w.m + fb * t, layer_mode(t, P.T), st));
  }
  float* e_atoms = atom_energy ? atom_energy : w.e_atoms;
  MP_TRY(fill_zero(w.flag, sizeof(int32_t), st));
  if (heads) {
    // every head reads the same last-layer features; E = sum_k lam_k E_k, and the one
    // reverse pass below starts from the lam-weighted sum of the heads' gradients
    if (!head_energy || !atom_energy) return arg_error("null head_energy/head_atom_energy");
    MP_TRY(dispatch_readout(P, heads->R, w.h, heads->wrT, heads->wout, e_atoms, st));
    for (int k = 0; k < heads->R; ++k)
      MP_TRY(launch_energy(e_atoms + (size_t)k * P.n, P.n, head_energy + k, w.flag, st));
    MP_TRY(launch_weighted_sum(head_energy, heads->lam, heads->R, energy, w.flag, st));
    MP_TRY(dispatch_readout_bwd(P, heads->R, w.h, heads->wrT, heads->wr, heads->wout, heads->lam, w.g_h, st));
  } else {
    MP_TRY(dispatch_readout(P, 1, w.h, m->wrT, m->wout, e_atoms, st));
    MP_TRY(launch_energy(e_atoms, P.n, energy, w.flag, st));
    MP_TRY(dispatch_readout_bwd(P, 1, w.h, m->wrT, m->wr, m->wout, nullptr, w.g_h, st));
  }
  // reverse pass through the layers
  MP_TRY(fill_zero(w.gd, sizeof(float) * (size_t)gd_floats(P), st));
  BwdArgs B{};
  B.g_m = w.g_m;
  B.g_ht = w.g_ht;
  B.g_q = w.g_q;
  B.ag = w.ag;
  B.gd = w.gd;
  B.gd_cap = P.cap;
  B.gd_half = gd_half_slots(P);
  for (int t = P.T - 1; t >= 0; --t) {
    A.ht = (char*)w.ht + fb * t;
    A.q = w.q + (size_t)t * P.n * P.C;
    A.mz = w.mz + (size_t)t * P.n * P.H * 2;
    B.m_saved = (char*)w.m + fb * t;
    MP_TRY(dispatch_layer_bwd(P, A, m->layers[t], B, w.g_h, layer_mode(t, P.T), t > 0, st));
  }
  MP_TRY(launch_forces(P, g, w.G, w.gd, perm, forces, w.flag, st));
  if (flag_out) *flag_out = w.flag;
  return MP_OK;
}
}  // namespace mdmp

extern "C" int mp_heads_create(const mp_model* m, int32_t n_heads, const float* wr, const float* wout,
                               const float* lam, mp_heads** out) {
  if (!m || !wr || !wout || !lam || !out) return arg_error("mp_heads_create: null argument");
  if (n_heads < 1 || n_heads > MP_MAX_HEADS) return arg_error("mp_heads_create: n_heads out of range");
  const int C = m->cfg.channels, R = n_heads;
  const size_t CC = (size_t)C * C;
  for (int k = 0; k < R; ++k)
    if (!std::isfinite(lam[k])) return arg_error("mp_heads_create: non-finite head weight");
  // device layout: [W_r per head, (out, in)][W_r^T per head, (in, out)][w_out per head][lam]
  std::vector<float> buf(2 * R * CC + (size_t)R * C + R);
  std::copy(wr, wr + R * CC, buf.begin());
  for (int k = 0; k < R; ++k)
    for (int o = 0; o < C; ++o)
      for (int i = 0; i < C; ++i) buf[R * CC + k * CC + (size_t)i * C + o] = wr[k * CC + (size_t)o * C + i];
  std::copy(wout, wout + (size_t)R * C, buf.begin() + 2 * R * CC);
  std::copy(lam, lam + R, buf.begin() + 2 * R * CC + (size_t)R * C);
  float* dev = nullptr;
  hipError_t e = hipMalloc((void**)&dev, sizeof(float) * buf.size());
  if (e != hipSuccess) {
    set_error(std::string("hipMalloc: ") + hipGetErrorString(e));
    return MP_ERR_HIP;
  }
  if (hipMemcpy(dev, buf.data(), sizeof(float) * buf.size(), hipMemcpyHostToDevice) != hipSuccess) {
    hipFree(dev);
    set_error("hipMemcpy of head weights failed");
    return MP_ERR_HIP;
  }
  mp_heads* h = new mp_heads();
  h->R = R;
  h->C = C;
  h->dev = dev;
  h->wr = dev;
  h->wrT = dev + R * CC;
  h->wout = dev + 2 * R * CC;
  h->lam = dev + 2 * R * CC + (size_t)R * C;
  *out = h;
  return MP_OK;
}

extern "C" int mp_heads_destroy(mp_heads* h) {
  if (!h) return MP_OK;
  hipFree(h->dev);
  delete h;
  return MP_OK;
}

extern "C" int mp_energy_forces_heads(const mp_model* m, const mp_heads* heads, const mp_graph* g,
                                      const int32_t* perm, double* head_energy, double* energy, float* forces,
                                      float* head_atom_energy, void* ws, size_t ws_bytes, hipStream_t st) {
  if (!g || !heads) return arg_error("null graph or heads");
  if (!m || heads->C != m->cfg.channels) return arg_error("heads were made for a model with other channels");
  if (!head_energy || !head_atom_energy) return arg_error("null head_energy/head_atom_energy");
  return ef_enqueue(m, g, g->n_edges, perm, energy, forces, head_atom_energy, ws, ws_bytes, nullptr, st, heads,
                    head_energy);
}

extern "C" int mp_energy_forces(const mp_model* m, const mp_graph* g, const int32_t* perm, double* energy,
                                float* forces, float* atom_energy, void* ws, size_t ws_bytes, hipStream_t st) {
  if (!g) return arg_error("null graph");
  return ef_enqueue(m, g, g->n_edges, perm, energy, forces, atom_energy, ws, ws_bytes, nullptr, st);
}

extern "C" int mp_energy_forces_status(const void* ws, hipStream_t st) {
  if (!ws) return arg_error("mp_energy_forces_status: null workspace");
  int32_t hflag = 0;
  MP_HIP(hipMemcpyAsync(&hflag, ws, sizeof(int32_t), hipMemcpyDeviceToHost, st));
  MP_HIP(hipStreamSynchronize(st));
  if (hflag) {
    set_error("non-finite energy or force");
    return MP_ERR_NUMERIC;
  }
  return MP_OK;
}
