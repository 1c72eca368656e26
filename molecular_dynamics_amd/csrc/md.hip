// NVE molecular dynamics with skin-triggered rebuilds and hipGraph replay.
//
// "Ab Initio Accuracy Beyond the Cutoff" (Abstract): a conservative neighbour
// skin preserves the graph's topology between updates, so each rebuild
// interval replays one captured graph; NVE energy drift measures fidelity.
// Velocity Verlet (textbook):
//   G_a: v += dt/2 a;  x += dt v;  flag = any |x - x_ref| > skin/2
//   host reads the 4-byte flag; if set: wrap + Hilbert re-sort + rebuild (not captured)
//   G_b: forces (the whole mp_energy_forces sequence);  a = F/m * 9.64853321e-3;
//        v += dt/2 a;  (KE, PE) in float64
// Langevin (NVT) steps use the BAOAB splitting (Leimkuhler & Matthews, "Rational
// construction of stochastic numerical methods for molecular sampling", 2013) in G_a:
//   v += dt/2 a;  x += dt/2 v;  v = c1 v + sqrt((1 - c1^2) kT/m) xi;  x += dt/2 v
// with c1 = exp(-gamma dt) and the caller's standard normals xi (input-atom order).
// Both graphs are captured once per edge-capacity bucket and replayed.  State
// arrays keep their addresses across rebuilds (they are permuted through a
// scratch copy), so the graphs stay valid until the capacity must grow.
#include <climits>
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "model.hpp"

namespace mdmp {

constexpr double kAcc = 9.64853321e-3;  // (eV/A)/amu -> A/fs^2
constexpr double kKe = 103.642696;      // amu (A/fs)^2 -> eV

__global__ void k_kick_drift(float* __restrict__ x, float* __restrict__ v, const float* __restrict__ a,
                             const float* __restrict__ xref, int n, float dt, float lim2,
                             int32_t* __restrict__ flag) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float d2 = 0.f;
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    float vv = v[3 * i + q] + 0.5f * dt * a[3 * i + q];
    v[3 * i + q] = vv;
    float xx = x[3 * i + q] + dt * vv;
    x[3 * i + q] = xx;
    float d = xx - xref[3 * i + q];
    d2 += d * d;
  }
  if (d2 > lim2) atomicOr(flag, 1);
}

__global__ void k_zero_flag(int32_t* flag) { *flag = 0; }

constexpr double kBoltz = 8.617333262e-5;  // eV/K

// B, A, O, A of one BAOAB step and the displacement flag.  The noise of this step is
// nz[0][(step * n + ids[i]) * 3 + q], step = *dstep (pointer and counter live in
// device memory so that a captured graph reads the current call's noise).
__global__ void k_baoab(float* __restrict__ x, float* __restrict__ v, const float* __restrict__ a,
                        const float* __restrict__ xref, const int32_t* __restrict__ ids,
                        const float* __restrict__ mass, int n, float dt, float c1, float kt_acc,
                        const float* const* __restrict__ nz, const int32_t* __restrict__ dstep, float lim2,
                        int32_t* __restrict__ flag) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float* xi = nz[0] + ((size_t)dstep[0] * n + ids[i]) * 3;
  const float sig = sqrtf((1.0f - c1 * c1) * kt_acc / mass[i]);
  float d2 = 0.f;
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    float vv = v[3 * i + q] + 0.5f * dt * a[3 * i + q];
    float xx = x[3 * i + q] + 0.5f * dt * vv;
    vv = c1 * vv + sig * xi[q];
    xx = xx + 0.5f * dt * vv;
    v[3 * i + q] = vv;
    x[3 * i + q] = xx;
    float d = xx - xref[3 * i + q];
    d2 += d * d;
  }
  if (d2 > lim2) atomicOr(flag, 1);
}

__global__ void k_step_inc(int32_t* dstep) { dstep[0] += 1; }

__global__ void k_set_noise(const float** nz, const float* p, int32_t* dstep) {
  nz[0] = p;
  dstep[0] = 0;
}

__global__ void k_accel_kick(const float* __restrict__ F, const float* __restrict__ mass, float* __restrict__ v,
                             float* __restrict__ a, int n, float dt, int kick) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float s = (float)kAcc / mass[i];
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    float aa = F[3 * i + q] * s;
    a[3 * i + q] = aa;
    if (kick) v[3 * i + q] += 0.5f * dt * aa;
  }
}

// (KE, PE) in float64, fixed summation order
__global__ __launch_bounds__(1024) void k_energies(const float* __restrict__ v, const float* __restrict__ mass,
                                                   int n, const double* __restrict__ epot, double* __restrict__ out) {
  __shared__ double sh[1024];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += 1024) {
    double v2 = (double)v[3 * i] * v[3 * i] + (double)v[3 * i + 1] * v[3 * i + 1] + (double)v[3 * i + 2] * v[3 * i + 2];
    s += (double)mass[i] * v2;
  }
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    out[0] = 0.5 * sh[0] * kKe;
    out[1] = epot[0];
  }
}

__global__ void k_set_input(const float* __restrict__ pos, const float* __restrict__ vel,
                            const int32_t* __restrict__ sp, const float* __restrict__ mps, int n,
                            float* __restrict__ x, float* __restrict__ v, int32_t* __restrict__ ids,
                            int32_t* __restrict__ spo, float* __restrict__ mass) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    x[3 * i + q] = pos[3 * i + q];
    v[3 * i + q] = vel[3 * i + q];
  }
  ids[i] = i;
  spo[i] = sp[i];
  mass[i] = mps[sp[i]];
}

// new slot s takes old slot perm[s]
__global__ void k_permute(const int32_t* __restrict__ perm, int n, const float* __restrict__ v_in,
                          const int32_t* __restrict__ ids_in, const float* __restrict__ m_in, float* __restrict__ v_out,
                          int32_t* __restrict__ ids_out, float* __restrict__ m_out) {
  int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= n) return;
  const int o = perm[s];
#pragma unroll
  for (int q = 0; q < 3; ++q) v_out[3 * s + q] = v_in[3 * o + q];
  ids_out[s] = ids_in[o];
  m_out[s] = m_in[o];
}

__global__ void k_unsort3(const float* __restrict__ src, const int32_t* __restrict__ ids, int n,
                          float* __restrict__ dst) {
  int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= n) return;
  const int o = ids[s];
#pragma unroll
  for (int q = 0; q < 3; ++q) dst[3 * o + q] = src[3 * s + q];
}

// minimum pair distance over the current list (min image, float32)
__global__ void k_min_dist(const float* __restrict__ x, const int32_t* __restrict__ row_ptr,
                           const int32_t* __restrict__ col, int n, float L, unsigned int* __restrict__ out) {
  int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= n) return;
  float best = INFINITY;
  for (int e = row_ptr[s]; e < row_ptr[s + 1]; ++e) {
    const int j = col[e];
    float d2 = 0.f;
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      float d = x[3 * j + q] - x[3 * s + q];
      d -= L * rintf(d / L);
      d2 += d * d;
    }
    best = fminf(best, d2);
  }
  atomicMin(out, __float_as_uint(sqrtf(best)));
}

}  // namespace mdmp

using namespace mdmp;

struct mp_md {
  const mp_model* model = nullptr;
  int32_t n = 0;
  float L = 0, skin = 0, dt = 0;
  hipStream_t st = nullptr;
  hipEvent_t ev = nullptr;
  // device state (slot order)
  float *x = nullptr, *v = nullptr, *a = nullptr, *xref = nullptr, *mass = nullptr, *F = nullptr, *mps = nullptr;
  int32_t *ids = nullptr, *sp = nullptr;
  // scratch for re-sorting
  float *x2 = nullptr, *v2 = nullptr, *m2 = nullptr;
  int32_t *ids2 = nullptr, *sp2 = nullptr, *perm = nullptr;
  // graph
  int32_t *row_ptr = nullptr, *col = nullptr, *rev = nullptr;
  int64_t cap = 0, n_edges = 0;
  void* nb_ws = nullptr;
  size_t nb_ws_bytes = 0;
  void* ef_ws = nullptr;
  size_t ef_ws_bytes = 0;
  double *epot = nullptr, *energies = nullptr;
  int32_t* dflag = nullptr;
  int32_t* hflag = nullptr;  // pinned [2]: displacement flag, non-finite flag of the last forces
  unsigned int* dmin = nullptr;
  hipGraphExec_t ga = nullptr, gb = nullptr;
  int64_t step = 0;
  int32_t n_rebuilds = 0, n_captures = 0;
  bool ready = false;
  bool graphs = true;  // replay the captured step graphs (else enqueue the kernels each step)
  // Langevin thermostat (BAOAB): on when gamma > 0
  bool nvt = false;
  float c1 = 1.0f, kt_acc = 0.0f;  // exp(-gamma dt); k_B T in amu (A/fs)^2
  const float** dnoise = nullptr;  // device: the current call's noise pointer
  int32_t* dstep = nullptr;        // device: step index within the current call
};

namespace {

template <class T>
int dalloc(T** p, size_t count) {
  MP_HIP(hipMalloc((void**)p, sizeof(T) * (count > 0 ? count : 1)));
  return MP_OK;
}

// the non-finite flag of the last force evaluation sits at the start of its workspace
int numeric_error(int64_t step) {
  set_error("non-finite energy or force at MD step " + std::to_string(step));
  return MP_ERR_NUMERIC;
}

void free_graphs(mp_md* md) {
  if (md->ga) hipGraphExecDestroy(md->ga);
  if (md->gb) hipGraphExecDestroy(md->gb);
  md->ga = md->gb = nullptr;
}

mp_graph graph_of(const mp_md* md) {
  mp_graph g{};
  g.n = md->n;
  g.box_L = md->L;
  g.pos = md->x;
  g.species = md->sp;
  g.row_ptr = md->row_ptr;
  g.col = md->col;
  g.rev = md->rev;
  g.n_edges = md->n_edges;
  return g;
}

int enqueue_forces(mp_md* md, bool kick, hipStream_t st) {
  mp_graph g = graph_of(md);
  g.n_edges = md->cap;  // kernels read row pointers from the device; the plan uses the capacity
  MP_TRY(ef_enqueue(md->model, &g, md->cap, nullptr, md->epot, md->F, nullptr, md->ef_ws, md->ef_ws_bytes, nullptr, st));
  k_accel_kick<<<cdiv(md->n, 256), 256, 0, st>>>(md->F, md->mass, md->v, md->a, md->n, md->dt, kick ? 1 : 0);
  k_energies<<<1, 1024, 0, st>>>(md->v, md->mass, md->n, md->epot, md->energies);
  MP_CHECK_LAUNCH();
  return MP_OK;
}

int grow(mp_md* md, int64_t need) {
  // capacity bucket: 1.1 x the need, rounded up to 2^20 edges
  int64_t cap = (int64_t)std::ceil(1.1 * (double)need);
  cap = ((cap + (1 << 20) - 1) >> 20) << 20;
  if (cap > INT_MAX) return arg_error("edge capacity beyond int32");
  free_graphs(md);
  if (md->col) hipFree(md->col);
  if (md->rev) hipFree(md->rev);
  if (md->ef_ws) hipFree(md->ef_ws);
  md->col = md->rev = nullptr;
  md->ef_ws = nullptr;
  MP_TRY(dalloc(&md->col, cap));
  MP_TRY(dalloc(&md->rev, cap));
  size_t b = 0;
  MP_TRY(mp_energy_forces_ws(md->model, md->n, cap, &b));
  MP_HIP(hipMalloc(&md->ef_ws, b));
  md->ef_ws_bytes = b;
  md->cap = cap;
  return MP_OK;
}

// wrap + re-sort all state along the Hilbert curve and rebuild the list
int rebuild(mp_md* md) {
  hipStream_t st = md->st;
  const int n = md->n;
  for (int attempt = 0; attempt < 2; ++attempt) {
    int64_t ne = 0;
    int rc = mp_build_neighbors(md->x, md->sp, n, md->L, md->model->cfg.cutoff, md->skin, md->perm, md->x2, md->sp2,
                                md->row_ptr, md->col, md->rev, md->cap, &ne, md->nb_ws, md->nb_ws_bytes, st);
    if (rc == MP_ERR_CAPACITY) {
      MP_TRY(grow(md, ne));
      continue;
    }
    MP_TRY(rc);
    md->n_edges = ne;
    k_permute<<<cdiv(n, 256), 256, 0, st>>>(md->perm, n, md->v, md->ids, md->mass, md->v2, md->ids2, md->m2);
    MP_CHECK_LAUNCH();
    MP_HIP(hipMemcpyAsync(md->x, md->x2, sizeof(float) * 3 * n, hipMemcpyDeviceToDevice, st));
    MP_HIP(hipMemcpyAsync(md->xref, md->x2, sizeof(float) * 3 * n, hipMemcpyDeviceToDevice, st));
    MP_HIP(hipMemcpyAsync(md->sp, md->sp2, sizeof(int32_t) * n, hipMemcpyDeviceToDevice, st));
    MP_HIP(hipMemcpyAsync(md->v, md->v2, sizeof(float) * 3 * n, hipMemcpyDeviceToDevice, st));
    MP_HIP(hipMemcpyAsync(md->ids, md->ids2, sizeof(int32_t) * n, hipMemcpyDeviceToDevice, st));
    MP_HIP(hipMemcpyAsync(md->mass, md->m2, sizeof(float) * n, hipMemcpyDeviceToDevice, st));
    md->n_rebuilds++;
    return MP_OK;
  }
  set_error("rebuild: capacity could not be satisfied");
  return MP_ERR_CAPACITY;
}

// first half-kick, drift (Langevin: B A O A) and the displacement flag
int enqueue_drift(mp_md* md, hipStream_t st) {
  k_zero_flag<<<1, 1, 0, st>>>(md->dflag);
  if (md->nvt) {
    k_baoab<<<cdiv(md->n, 256), 256, 0, st>>>(md->x, md->v, md->a, md->xref, md->ids, md->mass, md->n, md->dt,
                                               md->c1, md->kt_acc, md->dnoise, md->dstep,
                                               0.25f * md->skin * md->skin, md->dflag);
    k_step_inc<<<1, 1, 0, st>>>(md->dstep);
  } else {
    k_kick_drift<<<cdiv(md->n, 256), 256, 0, st>>>(md->x, md->v, md->a, md->xref, md->n, md->dt,
                                                    0.25f * md->skin * md->skin, md->dflag);
  }
  MP_CHECK_LAUNCH();
  return MP_OK;
}

int capture(mp_md* md) {
  free_graphs(md);
  hipStream_t st = md->st;
  hipGraph_t g = nullptr;
  MP_HIP(hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal));
  const int r1 = enqueue_drift(md, st);
  hipError_t e2 = hipStreamEndCapture(st, &g);
  if (r1 != MP_OK || e2 != hipSuccess) {
    if (g) hipGraphDestroy(g);
    set_error("capture of the drift graph failed");
    return MP_ERR_HIP;
  }
  MP_HIP(hipGraphInstantiate(&md->ga, g, nullptr, nullptr, 0));
  hipGraphDestroy(g);
  g = nullptr;
  MP_HIP(hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal));
  int rc = enqueue_forces(md, true, st);
  e2 = hipStreamEndCapture(st, &g);
  if (rc != MP_OK) {
    if (g) hipGraphDestroy(g);
    return rc;
  }
  if (e2 != hipSuccess) {
    set_error("capture of the force graph failed");
    return MP_ERR_HIP;
  }
  MP_HIP(hipGraphInstantiate(&md->gb, g, nullptr, nullptr, 0));
  hipGraphDestroy(g);
  md->n_captures++;
  return MP_OK;
}

void release(mp_md* md) {
  free_graphs(md);
  void* ps[] = {md->x, md->v, md->a, md->xref, md->mass, md->F, md->mps, md->ids, md->sp, md->x2, md->v2,
                md->m2, md->ids2, md->sp2, md->perm, md->row_ptr, md->col, md->rev, md->nb_ws, md->ef_ws,
                md->epot, md->energies, md->dflag, md->dmin, (void*)md->dnoise, md->dstep};
  for (void* p : ps)
    if (p) hipFree(p);
  if (md->hflag) hipHostFree(md->hflag);
  if (md->ev) hipEventDestroy(md->ev);
  if (md->st) hipStreamDestroy(md->st);
}

// the handle's stream waits for the caller's stream (and the reverse at the end)
int join(hipStream_t from, hipStream_t to, hipEvent_t ev) {
  MP_HIP(hipEventRecord(ev, from));
  MP_HIP(hipStreamWaitEvent(to, ev, 0));
  return MP_OK;
}

}  // namespace

extern "C" int mp_md_create(const mp_model* m, int32_t n, float box_L, float skin, float dt_fs,
                            const float* mass_per_species, mp_md** out) {
  if (!m || !out || !mass_per_species) return arg_error("mp_md_create: null argument");
  if (n < 2 || !(box_L > 0) || !(skin >= 0) || !(dt_fs > 0)) return arg_error("mp_md_create: bad sizes");
  if ((double)m->cfg.cutoff + skin >= 0.5 * (double)box_L) {
    set_error("mp_md_create: r_cut + skin must be < L/2");
    return MP_ERR_BOX;
  }
  for (int s = 0; s < m->cfg.n_species; ++s)
    if (!(mass_per_species[s] > 0)) return arg_error("mp_md_create: masses must be > 0");
  mp_md* md = new mp_md();
  md->model = m;
  md->n = n;
  md->L = box_L;
  md->skin = skin;
  md->dt = dt_fs;
  auto fail = [&](int rc) {
    release(md);
    delete md;
    return rc;
  };
  int rc = MP_OK;
#define MD_TRY(x)            \
  do {                       \
    rc = (x);                \
    if (rc != MP_OK) return fail(rc); \
  } while (0)
  if (hipStreamCreateWithFlags(&md->st, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&md->ev, hipEventDisableTiming) != hipSuccess) {
    set_error("mp_md_create: stream/event creation failed");
    return fail(MP_ERR_HIP);
  }
  MD_TRY(dalloc(&md->x, 3 * (size_t)n));
  MD_TRY(dalloc(&md->v, 3 * (size_t)n));
  MD_TRY(dalloc(&md->a, 3 * (size_t)n));
  MD_TRY(dalloc(&md->xref, 3 * (size_t)n));
  MD_TRY(dalloc(&md->F, 3 * (size_t)n));
  MD_TRY(dalloc(&md->mass, n));
  MD_TRY(dalloc(&md->mps, m->cfg.n_species));
  MD_TRY(dalloc(&md->ids, n));
  MD_TRY(dalloc(&md->sp, n));
  MD_TRY(dalloc(&md->x2, 3 * (size_t)n));
  MD_TRY(dalloc(&md->v2, 3 * (size_t)n));
  MD_TRY(dalloc(&md->m2, n));
  MD_TRY(dalloc(&md->ids2, n));
  MD_TRY(dalloc(&md->sp2, n));
  MD_TRY(dalloc(&md->perm, n));
  MD_TRY(dalloc(&md->row_ptr, n + 1));
  MD_TRY(dalloc(&md->epot, 1));
  MD_TRY(dalloc(&md->energies, 2));
  MD_TRY(dalloc(&md->dflag, 1));
  MD_TRY(dalloc(&md->dmin, 1));
  MD_TRY(dalloc(&md->dnoise, 1));
  MD_TRY(dalloc(&md->dstep, 1));
  if (hipHostMalloc((void**)&md->hflag, 2 * sizeof(int32_t), hipHostMallocDefault) != hipSuccess) {
    set_error("mp_md_create: pinned allocation failed");
    return fail(MP_ERR_HIP);
  }
  MD_TRY(mp_build_neighbors_ws(n, box_L, m->cfg.cutoff, skin, &md->nb_ws_bytes));
  if (hipMalloc(&md->nb_ws, md->nb_ws_bytes) != hipSuccess) {
    set_error("mp_md_create: workspace allocation failed");
    return fail(MP_ERR_HIP);
  }
  if (hipMemcpy(md->mps, mass_per_species, sizeof(float) * m->cfg.n_species, hipMemcpyHostToDevice) != hipSuccess) {
    set_error("mp_md_create: copy of masses failed");
    return fail(MP_ERR_HIP);
  }
  const double R = (double)m->cfg.cutoff + skin;
  MD_TRY(grow(md, (int64_t)(1.2 * n * ((double)n / ((double)box_L * box_L * box_L)) * 4.18879 * R * R * R) + 1024));
#undef MD_TRY
  *out = md;
  return MP_OK;
}

extern "C" int mp_md_set_state(mp_md* md, const float* pos, const float* vel, const int32_t* species, hipStream_t caller) {
  if (!md || !pos || !vel || !species) return arg_error("mp_md_set_state: null argument");
  MP_TRY(join(caller, md->st, md->ev));
  k_set_input<<<cdiv(md->n, 256), 256, 0, md->st>>>(pos, vel, species, md->mps, md->n, md->x, md->v, md->ids, md->sp,
                                                    md->mass);
  MP_CHECK_LAUNCH();
  const int64_t cap0 = md->cap;
  MP_TRY(rebuild(md));
  md->n_rebuilds = 0;
  if (md->graphs && (!md->gb || md->cap != cap0)) MP_TRY(capture(md));
  // first forces: a = F/m, no kick
  MP_TRY(enqueue_forces(md, false, md->st));
  md->step = 0;
  MP_HIP(hipMemcpyAsync(md->hflag + 1, md->ef_ws, sizeof(int32_t), hipMemcpyDeviceToHost, md->st));
  MP_HIP(hipStreamSynchronize(md->st));
  if (md->hflag[1]) return numeric_error(0);
  md->ready = true;
  return MP_OK;
}

namespace {
int run_steps(mp_md* md, int32_t n_steps, double* e_log, hipStream_t caller) {
  MP_TRY(join(caller, md->st, md->ev));
  if (md->graphs && !md->gb) MP_TRY(capture(md));
  for (int32_t s = 0; s < n_steps; ++s) {
    if (md->graphs) {
      MP_HIP(hipGraphLaunch(md->ga, md->st));
    } else {
      MP_TRY(enqueue_drift(md, md->st));
    }
    // one read per step: the displacement flag, and the forces of the previous step
    MP_HIP(hipMemcpyAsync(md->hflag, md->dflag, sizeof(int32_t), hipMemcpyDeviceToHost, md->st));
    MP_HIP(hipMemcpyAsync(md->hflag + 1, md->ef_ws, sizeof(int32_t), hipMemcpyDeviceToHost, md->st));
    MP_HIP(hipStreamSynchronize(md->st));
    if (md->hflag[1]) return numeric_error(md->step);
    if (*md->hflag) {
      const int64_t cap0 = md->cap;
      MP_TRY(rebuild(md));
      if (md->graphs && md->cap != cap0) MP_TRY(capture(md));
    }
    if (md->graphs) {
      MP_HIP(hipGraphLaunch(md->gb, md->st));
    } else {
      MP_TRY(enqueue_forces(md, true, md->st));
    }
    if (e_log) MP_HIP(hipMemcpyAsync(e_log + 2 * (size_t)s, md->energies, 2 * sizeof(double), hipMemcpyDeviceToDevice, md->st));
    md->step++;
  }
  if (n_steps > 0) {
    // the last step's forces
    MP_HIP(hipMemcpyAsync(md->hflag + 1, md->ef_ws, sizeof(int32_t), hipMemcpyDeviceToHost, md->st));
    MP_HIP(hipStreamSynchronize(md->st));
    if (md->hflag[1]) return numeric_error(md->step);
  }
  MP_TRY(join(md->st, caller, md->ev));
  return MP_OK;
}
}  // namespace

extern "C" int mp_md_step(mp_md* md, int32_t n_steps, double* e_log, hipStream_t caller) {
  if (!md) return arg_error("mp_md_step: null handle");
  if (!md->ready) {
    set_error("mp_md_step: call mp_md_set_state first");
    return MP_ERR_STATE;
  }
  if (md->nvt) {
    set_error("mp_md_step: the Langevin thermostat is on; use mp_md_step_nvt");
    return MP_ERR_STATE;
  }
  if (n_steps < 0) return arg_error("mp_md_step: n_steps < 0");
  return run_steps(md, n_steps, e_log, caller);
}

extern "C" int mp_md_set_langevin(mp_md* md, float temperature_K, float gamma_per_ps) {
  if (!md) return arg_error("mp_md_set_langevin: null handle");
  if (!(temperature_K >= 0) || !(gamma_per_ps >= 0) || !std::isfinite(temperature_K) || !std::isfinite(gamma_per_ps))
    return arg_error("mp_md_set_langevin: temperature and friction must be finite and >= 0");
  const bool nvt = gamma_per_ps > 0;
  if (nvt != md->nvt) free_graphs(md);  // the drift graph changes
  md->nvt = nvt;
  md->c1 = (float)std::exp(-(double)gamma_per_ps * 1e-3 * (double)md->dt);
  md->kt_acc = (float)(kBoltz * (double)temperature_K * kAcc);
  return MP_OK;
}

extern "C" int mp_md_step_nvt(mp_md* md, int32_t n_steps, const float* noise, double* e_log, hipStream_t caller) {
  if (!md) return arg_error("mp_md_step_nvt: null handle");
  if (!md->ready) {
    set_error("mp_md_step_nvt: call mp_md_set_state first");
    return MP_ERR_STATE;
  }
  if (!md->nvt) {
    set_error("mp_md_step_nvt: no thermostat (mp_md_set_langevin with gamma > 0 first)");
    return MP_ERR_STATE;
  }
  if (n_steps < 0) return arg_error("mp_md_step_nvt: n_steps < 0");
  if (n_steps > 0 && !noise) return arg_error("mp_md_step_nvt: null noise");
  MP_TRY(join(caller, md->st, md->ev));
  k_set_noise<<<1, 1, 0, md->st>>>(md->dnoise, noise, md->dstep);
  MP_CHECK_LAUNCH();
  MP_TRY(join(md->st, caller, md->ev));
  return run_steps(md, n_steps, e_log, caller);
}

extern "C" int mp_md_use_graphs(mp_md* md, int32_t enable) {
  if (!md) return arg_error("mp_md_use_graphs: null handle");
  md->graphs = enable != 0;
  return MP_OK;
}

extern "C" int mp_md_get_state(mp_md* md, float* pos, float* vel, int64_t* step, int32_t* n_rebuilds,
                               int32_t* n_captures, float* min_pair_dist, hipStream_t caller) {
  if (!md) return arg_error("mp_md_get_state: null handle");
  MP_TRY(join(caller, md->st, md->ev));
  if (pos) k_unsort3<<<cdiv(md->n, 256), 256, 0, md->st>>>(md->x, md->ids, md->n, pos);
  if (vel) k_unsort3<<<cdiv(md->n, 256), 256, 0, md->st>>>(md->v, md->ids, md->n, vel);
  MP_CHECK_LAUNCH();
  if (min_pair_dist) {
    unsigned int init = 0x7f800000u;  // +inf
    MP_HIP(hipMemcpyAsync(md->dmin, &init, sizeof(init), hipMemcpyHostToDevice, md->st));
    k_min_dist<<<cdiv(md->n, 256), 256, 0, md->st>>>(md->x, md->row_ptr, md->col, md->n, md->L, md->dmin);
    MP_CHECK_LAUNCH();
    unsigned int h = 0;
    MP_HIP(hipMemcpyAsync(&h, md->dmin, sizeof(h), hipMemcpyDeviceToHost, md->st));
    MP_HIP(hipStreamSynchronize(md->st));
    std::memcpy(min_pair_dist, &h, 4);
  }
  if (step) *step = md->step;
  if (n_rebuilds) *n_rebuilds = md->n_rebuilds;
  if (n_captures) *n_captures = md->n_captures;
  MP_TRY(join(md->st, caller, md->ev));
  return MP_OK;
}

extern "C" int mp_md_destroy(mp_md* md) {
  if (!md) return MP_OK;
  if (md->st) hipStreamSynchronize(md->st);
  release(md);
  delete md;
  return MP_OK;
}
