/* mdmp.h -- C ABI of libmdmp: energy and forces of an equivariant
 * message-passing attention potential over a skin-padded radius graph, on
 * one AMD MI355X (gfx950).
 *
 * The operations follow "Ab Initio Accuracy Beyond the Cutoff: Distributed
 * Message-Passing Equivariant Attention at Tens-of-Millions-of-Atom Scale"
 * (Abstract): atoms are ordered along a space-filling curve, a conservative
 * neighbour skin keeps the graph fixed between rebuilds, stacked equivariant
 * attention layers give the energy, forces come from back-propagation, and
 * molecular dynamics replays one captured graph per rebuild interval.
 *
 * Conventions shared by every call
 *  - Return value: MP_OK (0) or a negative MP_ERR_* code.  No C++ exception
 *    crosses this boundary.  mp_last_error() returns a thread-local message
 *    describing the last failure on the calling thread.
 *  - Array arguments named "device" are device pointers owned by the caller.
 *    The library never frees them and never keeps them beyond the call,
 *    except inside an mp_md handle, which owns its own state.
 *  - Work is enqueued on the caller's HIP stream.  Host synchronisation
 *    happens only where a call says so.
 *  - Units: A, eV, amu, fs.  Positions are float32 [n][3] (x, y, z).
 *  - A handle is used from one stream at a time.
 */
#ifndef MDMP_H
#define MDMP_H

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MP_OK 0
#define MP_ERR_ARG (-1)      /* invalid argument (null pointer, bad size, unsupported config) */
#define MP_ERR_BOX (-2)      /* r_cut + skin >= L/2: minimum image is not unique */
#define MP_ERR_CAPACITY (-3) /* edge capacity too small; *n_edges holds the required size */
#define MP_ERR_HIP (-4)      /* a HIP runtime call failed; the message names it */
#define MP_ERR_NUMERIC (-5)  /* a non-finite energy or force was produced */
#define MP_ERR_STATE (-6)    /* handle misuse (e.g. stepping before set_state) */

int mp_version(void);
const char* mp_last_error(void);

/* ---------------------------------------------------------------- model ----
 * The potential (one layer is described for layer t; h_i^l in R^{C x (2l+1)}):
 *   ht_i^l = W_v^l h_i^l,  q_i = W_q h_i^0
 *   w_e[p,c] = u(r) (W_2 SiLU(W_1 B(r)))[p*C + c]             radial MLP
 *   v_e^{l3}[c,m3] = sum_p w_e[p,c] sum CG_p[m1,m2,m3] ht_j^{l1}[c,m1] Y_{l2,m2}(rhat)
 *   a_e^k = d_h^{-1/2} sum_{c in head k} q_i[c] v_e^0[c]
 *   alpha_e^k = u(r_e) exp(a_e^k - M_i^k) / sum_{e' in row i} u(r_e') exp(a_e'^k - M_i^k)
 *   m_i^l = sum_e alpha_e^{k(c)} v_e^l;   h^0 += SiLU(W_o^0 m^0);
 *   h^l += sigmoid(W_g m^0)[(l-1)C + c] * (W_o^l m^l)      (l >= 1)
 * with edge e = (i <- j), r_ij = x_j - x_i (minimum image), B the Bessel basis
 * sqrt(2/r_c) sin(n pi r/r_c)/r, u the p = 6 polynomial envelope, Y the
 * orthonormal real spherical harmonics and CG the real Clebsch-Gordan
 * tensors of all triangle paths (l1, l2, l3) <= lmax.  Energy:
 * E = sum_i w_out . SiLU(W_r h_i^0).  The equivariant-attention layer and
 * the Bessel/envelope radial basis are the forms named in the Tessera
 * abstract and in "Exascale Multi-Task Graph Foundation Models" (Table IV).
 *
 * feat_dtype 0: features and all arithmetic float32.  feat_dtype 1: features
 * h, ht, m stored as bfloat16; the dense products (per-atom linears and both
 * radial-MLP layers) take bf16 operands with float32 accumulation, and the
 * radial MLP's output w' of a tile (before the envelope factor u) is held as
 * bfloat16; geometry, tensor product, softmax and gates stay float32, as do
 * all sums ("Unlocking Tensor Core Performance", section "Choosing a
 * Precision Strategy").  The energy is always accumulated in float64. */
typedef struct {
  int32_t n_species;
  int32_t channels;      /* C: 16, 32, 64 or 128 */
  int32_t lmax;          /* 1 or 2 */
  int32_t n_bessel;      /* must be 8 */
  int32_t radial_hidden; /* must be 64 */
  int32_t heads;         /* H, divides C; C/H a power of two, at most 32 */
  int32_t layers;        /* T >= 1 */
  int32_t feat_dtype;    /* 0 = float32, 1 = bfloat16 features */
  float cutoff;          /* r_c in A */
} mp_model_config;

typedef struct mp_model mp_model;

/* Number of float32 weights the configuration needs.  Blob layout, each
 * matrix row-major [out][in]: E_emb [S][C]; per layer: W_1 [64][8],
 * W_2 [P*C][64] (row p*C + c), W_q [C][C], W_v^0..lmax [C][C],
 * W_o^0..lmax [C][C], W_g [lmax*C][C] (row (l-1)*C + c); then W_r [C][C],
 * w_out [1][C].  P = 5 (lmax 1) or 15 (lmax 2). */
int mp_model_num_weights(const mp_model_config* cfg, int64_t* n);

/* Copies the host weight blob to the device (bf16 copies for feat_dtype 1,
 * and W_2, W_2^T once more per layer in the order the edge kernels read their
 * matrix-core fragments, a few MB per layer) and builds the CG tables.  *out
 * owns device memory; free with mp_model_destroy.  Synchronous. */
int mp_model_create(const mp_model_config* cfg, const float* host_weights, int64_t n_weights,
                    mp_model** out);
int mp_model_destroy(mp_model* m);

/* Host-only: the library's real CG table for lmax (1 or 2), as rows of
 * (l1, l2, l3, m1+l1, m2+l2, m3+l3, value) float64, path order then
 * lexicographic (m1, m2, m3).  *n_rows receives the row count (137 for
 * lmax 2); rows beyond cap are not written. */
int mp_cg_table(int32_t lmax, double* out_rows7, int64_t cap, int64_t* n_rows);

/* ------------------------------------------------------------ neighbours --
 * Tessera abstract: atoms sorted along a space-filling curve; a conservative
 * skin; a three-level neighbour search.  Levels here: (1) Hilbert order of
 * the atoms, (2) cell list of side >= R = r_c + skin, (3) exact pair test.
 * The result is defined bit for bit:
 *  wrap   w = x - L floor(x/L) in float64 (no contraction), fixed up once
 *         each way into [0, L), rounded to float32; a float32 value equal
 *         to L becomes 0.
 *  order  key = 30-bit Hilbert index (Skilling's transpose algorithm, 10 bits
 *         per axis, x most significant) of g_a = min(1023,
 *         floor(x_a * 1024.0 / L)) in float64; stable by (key, input index).
 *  pairs  float64 d_a = P_t,a - P_s,a, one -L/+L shift when |d_a| > L/2,
 *         D = (dx*dx + dy*dy) + dz*dz; pair iff D < ((double)r_c + skin)^2.
 *  CSR    rows ascending, no self pairs, full directed list (int32);
 *         rev[e] is the position of (t -> s) for e = (s -> t).
 * Inputs (device): pos [n][3], species [n].  Outputs (device): perm [n]
 * (perm[s] = input index of sorted slot s), pos_sorted [n][3] (wrapped),
 * species_sorted [n], row_ptr [n+1], col [capacity], rev [capacity].
 * *n_edges (host) receives the edge count; if it exceeds capacity the call
 * returns MP_ERR_CAPACITY after writing perm/pos_sorted/species_sorted/
 * row_ptr but not col/rev.  ws: device scratch of at least
 * mp_build_neighbors_ws bytes.  Host sync: once, to read the edge count.
 * Errors: MP_ERR_BOX when r_c + skin >= L/2; MP_ERR_ARG when a row exceeds
 * 1024 neighbours or n < 2. */
int mp_build_neighbors_ws(int32_t n, float box_L, float cutoff, float skin, size_t* bytes);

/* Many small structures without periodic images in one graph (for
 * throughput on batches of molecules, "Exascale Multi-Task Graph Foundation
 * Models", Table XV reports structures per second): the atoms of structure b
 * are pos[struct_ptr[b] .. struct_ptr[b+1]-1] (device, int32 [n_struct+1],
 * struct_ptr[0] = 0, ascending, struct_ptr[n_struct] = n), and each atom's
 * neighbours are the atoms of its own structure closer than r_cut + skin
 * (float64, the operation order above without the image shift).  The slots
 * are the input order (no sort, no perm); row_ptr [n+1], col, rev as for
 * mp_build_neighbors.  The graph for the other calls is {n, box_L = 0, pos,
 * species, row_ptr, col, rev, n_edges}.  Host sync: once (edge count);
 * MP_ERR_CAPACITY with *n_edges set as above.  ws: at least
 * mp_build_neighbors_batched_ws bytes. */
int mp_build_neighbors_batched_ws(int32_t n, int32_t n_struct, size_t* bytes);
int mp_build_neighbors_batched(const float* pos, int32_t n, const int32_t* struct_ptr, int32_t n_struct,
                               float cutoff, float skin, int32_t* row_ptr, int32_t* col, int32_t* rev,
                               int64_t capacity, int64_t* n_edges, void* ws, size_t ws_bytes, hipStream_t stream);
/* energies[b] = sum of atom_energy over structure b (device; float64, fixed
 * order), for the atom energies of mp_energy_forces on a batched graph. */
int mp_structure_energies(const float* atom_energy, const int32_t* struct_ptr, int32_t n_struct, double* energies,
                          hipStream_t stream);

/* Atom orders for mp_build_neighbors_ordered.  The Tessera abstract ("Ab Initio
 * Accuracy Beyond the Cutoff", Abstract) sorts atoms along a space-filling
 * curve and compares the neighbour-search cost of its curve with Morton order;
 * MP_ORDER_INPUT keeps the caller's order (no locality), for the same
 * comparison.  Any order gives the same energy and (un-permuted) forces. */
#define MP_ORDER_HILBERT 0 /* Skilling's Hilbert curve, 10 bits per axis (mp_build_neighbors) */
#define MP_ORDER_MORTON 1  /* Z-order: the cell-coordinate bits interleaved, x most significant */
#define MP_ORDER_INPUT 2   /* perm = identity */
int mp_build_neighbors(const float* pos, const int32_t* species, int32_t n, float box_L, float cutoff,
                       float skin, int32_t* perm, float* pos_sorted, int32_t* species_sorted,
                       int32_t* row_ptr, int32_t* col, int32_t* rev, int64_t capacity, int64_t* n_edges,
                       void* ws, size_t ws_bytes, hipStream_t stream);
/* mp_build_neighbors with the atom order chosen by `order` (MP_ORDER_*): slots
 * follow that order instead of the Hilbert curve; the rest is identical
 * (mp_build_neighbors is this call with MP_ORDER_HILBERT).  MP_ERR_ARG for an
 * unknown order. */
int mp_build_neighbors_ordered(const float* pos, const int32_t* species, int32_t n, float box_L, float cutoff,
                               float skin, int32_t order, int32_t* perm, float* pos_sorted,
                               int32_t* species_sorted, int32_t* row_ptr, int32_t* col, int32_t* rev,
                               int64_t capacity, int64_t* n_edges, void* ws, size_t ws_bytes, hipStream_t stream);

/* A neighbour graph in sorted-slot order, as produced by mp_build_neighbors
 * (all pointers device).  Positions may be unwrapped drifts of the wrapped
 * ones: edge vectors use d -= L * rint(d / L).  box_L = 0 marks an open
 * boundary (no image shift), as produced by mp_build_neighbors_batched. */
typedef struct {
  int32_t n;
  float box_L;
  const float* pos;          /* [n][3] */
  const int32_t* species;    /* [n] */
  const int32_t* row_ptr;    /* [n+1] */
  const int32_t* col;        /* [n_edges] */
  const int32_t* rev;        /* [n_edges] */
  int64_t n_edges;
} mp_graph;

/* -------------------------------------------------------------- one layer --
 * Applies layer `layer` (0-based) to h_in, writing h_out (device, [n][K][C],
 * K = (lmax+1)^2, k = l^2 + m + l, channel fastest; float32 or bf16 bits per
 * feat_dtype).  h_in and h_out must not overlap and must be 16-byte aligned
 * (MP_ERR_ARG otherwise).  ws: at least mp_layer_forward_ws bytes.  No host
 * sync. */
int mp_layer_forward_ws(const mp_model* m, int32_t n, int64_t n_edges, size_t* bytes);
int mp_layer_forward(const mp_model* m, int32_t layer, const mp_graph* g, const void* h_in, void* h_out,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* Embedding of layer 0's input: h^0 = E_emb[species], h^{l>0} = 0.  h_out as
 * for mp_layer_forward (16-byte aligned). */
int mp_embed(const mp_model* m, const mp_graph* g, void* h_out, hipStream_t stream);

/* ------------------------------------------------------- energy + forces --
 * Full stack of layers, energy and forces F = -dE/dx by one reverse pass
 * (Tessera abstract: force back-propagation through the layers;
 * "Exascale Multi-Task Graph Foundation Models", Fig. 5: one backward pass
 * gives the forces).  Outputs (device): *energy (float64), forces [n][3]
 * float32 in input order when perm != NULL (forces[perm[s]] = F_s), else in
 * slot order; atom_energy [n] float32 (slot order) if not NULL.  The
 * backward scatter is deterministic (no floating-point atomics): repeated
 * calls give identical bits.  ws: at least mp_energy_forces_ws bytes.  No
 * host sync: the call only enqueues work (errors returned are argument and
 * launch errors).  A non-finite energy or force sets a 4-byte flag at the
 * start of ws, which mp_energy_forces_status reads. */
int mp_energy_forces_ws(const mp_model* m, int32_t n, int64_t n_edges, size_t* bytes);
int mp_energy_forces(const mp_model* m, const mp_graph* g, const int32_t* perm, double* energy,
                     float* forces, float* atom_energy, void* ws, size_t ws_bytes, hipStream_t stream);
/* Waits for `stream` (host sync) and returns MP_ERR_NUMERIC if the last
 * mp_energy_forces or mp_energy_forces_heads call on workspace ws produced a
 * non-finite energy or force, else MP_OK. */
int mp_energy_forces_status(const void* ws, hipStream_t stream);

/* For callers that cannot allocate device memory (work being captured into a
 * graph, tight serving loops, harnesses that forbid allocation): mp_energy_forces
 * with its workspace in a device array of the library, MP_NOALLOC_SCRATCH_BYTES
 * per GPU, held from the library's first use on that GPU until the process
 * ends.  Same outputs and kernels as mp_energy_forces (identical bits for the
 * same graph); no allocation, no host sync.  nonfinite (device int32,
 * nullable) receives 1 if the energy or a force is non-finite, else 0.
 * MP_ERR_ARG when the graph needs more workspace than the array holds
 * (mp_energy_forces_ws reports the need).  Every call on one GPU shares that
 * GPU's array: calls that overlap in time on one GPU (other streams, other
 * threads) race and must not be made. */
#define MP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int mp_energy_forces_noalloc(const mp_model* m, const mp_graph* g, const int32_t* perm, double* energy,
                             float* forces, float* atom_energy, int32_t* nonfinite, hipStream_t stream);

/* ------------------------------------------------ several readout heads ---
 * "Exascale Multi-Task Graph Foundation Models", Fig. 5 (fused gradient
 * inference): the encoder runs once, R readout heads read its output, their
 * energies are combined into a weighted sum, and one reverse pass gives the
 * forces of that sum.  Here head k has its own readout (W_r^k [C][C] (out,
 * in), w_out^k [C]) on the last layer's features:
 *   E_k = sum_i w_out^k . SiLU(W_r^k h_i^0),   E = sum_k lam_k E_k,
 *   F = -dE/dx.
 * mp_heads_create copies host arrays wr [R][C][C], wout [R][C], lam [R]
 * (finite) to the device; 1 <= R <= MP_MAX_HEADS; C is the model's channel
 * count.  The handle is freed by mp_heads_destroy and may be shared by
 * calls on one model's graphs. */
#define MP_MAX_HEADS 64
typedef struct mp_heads mp_heads;
int mp_heads_create(const mp_model* m, int32_t n_heads, const float* wr, const float* wout, const float* lam,
                    mp_heads** out);
int mp_heads_destroy(mp_heads* heads);
/* mp_energy_forces with the heads' readouts in place of the model's own.
 * Outputs (device): head_energy [R] float64 (each head's E_k, fixed-order
 * sum), *energy = sum_k lam_k E_k (float64, in head order), forces [n][3] of
 * that sum (input order if perm != NULL, as in mp_energy_forces),
 * head_atom_energy [R][n] float32 in slot order (required: it holds the
 * per-head atom energies).  ws: mp_energy_forces_ws bytes.  MP_ERR_ARG if
 * the heads were made for another channel count.  No host sync; the
 * non-finite flag as in mp_energy_forces (mp_energy_forces_status).  With R = 1, lam = 1 and the model's own W_r, w_out the
 * results equal mp_energy_forces bit for bit. */
int mp_energy_forces_heads(const mp_model* m, const mp_heads* heads, const mp_graph* g, const int32_t* perm,
                           double* head_energy, double* energy, float* forces, float* head_atom_energy, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- MD -------
 * NVE velocity Verlet with skin-triggered rebuilds (Tessera abstract: a
 * conservative skin lets each rebuild interval replay as one captured
 * graph).  Per step: v += dt/2 a; x += dt v; if max_i |x_i - x_i^ref| >
 * skin/2: wrap, re-sort all state along the Hilbert curve and rebuild;
 * a = F/m * 9.64853321e-3; v += dt/2 a; energies logged in float64.  The
 * kernels of a step are captured once into hipGraphs and replayed until a
 * rebuild needs more edge capacity.  The handle owns all device state. */
typedef struct mp_md mp_md;
/* mass_per_species: host [n_species] amu. */
int mp_md_create(const mp_model* m, int32_t n, float box_L, float skin, float dt_fs,
                 const float* mass_per_species, mp_md** out);
/* pos, vel (A/fs), species: device, input order.  Builds the first list and
 * the first forces.  Host sync.  MP_ERR_NUMERIC if those forces or the
 * energy are non-finite. */
int mp_md_set_state(mp_md* md, const float* pos, const float* vel, const int32_t* species,
                    hipStream_t stream);
/* Advances n_steps.  e_log (device, nullable): [n_steps][2] float64 of
 * (kinetic, potential) after each step.  Host syncs: one read of two 4-byte
 * flags per step (the rebuild decision and the non-finite flag of the
 * previous step's forces) and one at the end of the call (the last step's
 * forces).  MP_ERR_NUMERIC at the first non-finite energy or force; the
 * state is then that of the step that produced it. */
int mp_md_step(mp_md* md, int32_t n_steps, double* e_log, hipStream_t stream);
/* enable = 0: later steps enqueue their kernels one by one instead of replaying
 * the captured graphs (the same kernels in the same order, so the same bits);
 * enable = 1 (the default) replays graphs.  For the comparison of graph reuse
 * with eager launches ("Ab Initio Accuracy Beyond the Cutoff", Abstract: graph
 * reuse and full-step time). */
int mp_md_use_graphs(mp_md* md, int32_t enable);
/* Langevin thermostat (NVT), BAOAB splitting (Leimkuhler & Matthews 2013): per
 * step v += dt/2 a; x += dt/2 v; v = c1 v + sqrt((1 - c1^2) k_B T / m) xi;
 * x += dt/2 v; [rebuild check]; forces; v += dt/2 a, with c1 = exp(-gamma dt),
 * k_B = 8.617333262e-5 eV/K.  The Tessera abstract ("Ab Initio Accuracy
 * Beyond the Cutoff", Abstract) runs its capsid in NVT without naming the
 * thermostat; this is the plain reading.  gamma_per_ps > 0 turns it on (then
 * only mp_md_step_nvt steps), 0 turns it off; MP_ERR_ARG for negative or
 * non-finite values.  Host only; takes effect at the next step call. */
int mp_md_set_langevin(mp_md* md, float temperature_K, float gamma_per_ps);
/* As mp_md_step, with the thermostat on.  noise (device, float32,
 * [n_steps][n][3], input-atom order, caller-owned, read during the call
 * only): the standard normal deviates xi of each step, drawn by the caller
 * (so that any implementation can be given the same ones).  MP_ERR_STATE
 * without the thermostat or before mp_md_set_state. */
int mp_md_step_nvt(mp_md* md, int32_t n_steps, const float* noise, double* e_log, hipStream_t stream);
/* pos, vel (device [n][3], input order; nullable), counters (host, nullable). */
int mp_md_get_state(mp_md* md, float* pos, float* vel, int64_t* step, int32_t* n_rebuilds,
                    int32_t* n_captures, float* min_pair_dist, hipStream_t stream);
int mp_md_destroy(mp_md* md);

/* ------------------------------------------------------------ profiling ----
 * Optional kernel timing with hipEvents recorded on the launching stream
 * around the named launches: "build_neighbors", "geometry", "edge_fwd",
 * "edge_bwd_recv", "edge_bwd_send", "forces".  Off by default; recording is
 * skipped while a stream is being captured.  mp_profile_read synchronises the
 * recorded events and returns the summed time and the launch count for one
 * name since the last reset.  Host-side registry, not thread-safe across
 * concurrent streams. */
int mp_profile_enable(int on);
int mp_profile_reset(void);
int mp_profile_read(const char* name, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* MDMP_H */
