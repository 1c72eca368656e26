"""ctypes binding of libmdmp (the C ABI in include/mdmp.h).

Argument marshalling only: every step of the path runs in the HIP library.
PyTorch supplies device memory and the current stream.  Importing this module
fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmdmp.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libmdmp.so not found at {LIB_PATH}; run `python -m molecular_dynamics_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

ORDERS = {"hilbert": 0, "morton": 1, "input": 2}  # MP_ORDER_* of mdmp.h

NOALLOC_SCRATCH_BYTES = 64 << 20  # MP_NOALLOC_SCRATCH_BYTES of mdmp.h

MP_OK, MP_ERR_ARG, MP_ERR_BOX, MP_ERR_CAPACITY, MP_ERR_HIP, MP_ERR_NUMERIC, MP_ERR_STATE = 0, -1, -2, -3, -4, -5, -6
_NAMES = {-1: "MP_ERR_ARG", -2: "MP_ERR_BOX", -3: "MP_ERR_CAPACITY", -4: "MP_ERR_HIP", -5: "MP_ERR_NUMERIC",
          -6: "MP_ERR_STATE"}

EXPORTS = ["mp_version", "mp_last_error", "mp_model_num_weights", "mp_model_create", "mp_model_destroy",
           "mp_cg_table", "mp_build_neighbors_ws", "mp_build_neighbors", "mp_build_neighbors_ordered",
           "mp_build_neighbors_batched_ws", "mp_build_neighbors_batched", "mp_structure_energies",
           "mp_layer_forward_ws",
           "mp_layer_forward", "mp_embed", "mp_energy_forces_ws", "mp_energy_forces", "mp_energy_forces_status",
           "mp_energy_forces_noalloc", "mp_heads_create",
           "mp_heads_destroy", "mp_energy_forces_heads", "mp_md_create",
           "mp_md_set_state", "mp_md_step", "mp_md_use_graphs", "mp_md_set_langevin", "mp_md_step_nvt",
           "mp_md_get_state", "mp_md_destroy",
           "mp_profile_enable",
           "mp_profile_reset", "mp_profile_read"]


class MPError(RuntimeError):
    def __init__(self, code, where):
        msg = _lib.mp_last_error().decode(errors="replace")
        super().__init__(f"{where}: {_NAMES.get(code, code)}: {msg}")
        self.code = code


class mp_model_config(ctypes.Structure):
    _fields_ = [("n_species", ctypes.c_int32), ("channels", ctypes.c_int32), ("lmax", ctypes.c_int32),
                ("n_bessel", ctypes.c_int32), ("radial_hidden", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("layers", ctypes.c_int32), ("feat_dtype", ctypes.c_int32), ("cutoff", ctypes.c_float)]


class mp_graph(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("box_L", ctypes.c_float), ("pos", ctypes.c_void_p),
                ("species", ctypes.c_void_p), ("row_ptr", ctypes.c_void_p), ("col", ctypes.c_void_p),
                ("rev", ctypes.c_void_p), ("n_edges", ctypes.c_int64)]


_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_P = ctypes.POINTER
_sig = {
    "mp_version": ([], ctypes.c_int),
    "mp_last_error": ([], ctypes.c_char_p),
    "mp_model_num_weights": ([_P(mp_model_config), _P(_i64)], ctypes.c_int),
    "mp_model_create": ([_P(mp_model_config), _vp, _i64, _P(_vp)], ctypes.c_int),
    "mp_model_destroy": ([_vp], ctypes.c_int),
    "mp_cg_table": ([_i32, _vp, _i64, _P(_i64)], ctypes.c_int),
    "mp_build_neighbors_ws": ([_i32, _f32, _f32, _f32, _P(_sz)], ctypes.c_int),
    "mp_build_neighbors": ([_vp, _vp, _i32, _f32, _f32, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _P(_i64), _vp,
                            _sz, _vp], ctypes.c_int),
    "mp_build_neighbors_ordered": ([_vp, _vp, _i32, _f32, _f32, _f32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i64,
                                    _P(_i64), _vp, _sz, _vp], ctypes.c_int),
    "mp_build_neighbors_batched_ws": ([_i32, _i32, _P(_sz)], ctypes.c_int),
    "mp_build_neighbors_batched": ([_vp, _i32, _vp, _i32, _f32, _f32, _vp, _vp, _vp, _i64, _P(_i64), _vp, _sz, _vp],
                                   ctypes.c_int),
    "mp_structure_energies": ([_vp, _vp, _i32, _vp, _vp], ctypes.c_int),
    "mp_layer_forward_ws": ([_vp, _i32, _i64, _P(_sz)], ctypes.c_int),
    "mp_layer_forward": ([_vp, _i32, _P(mp_graph), _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "mp_embed": ([_vp, _P(mp_graph), _vp, _vp], ctypes.c_int),
    "mp_energy_forces_ws": ([_vp, _i32, _i64, _P(_sz)], ctypes.c_int),
    "mp_energy_forces": ([_vp, _P(mp_graph), _vp, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "mp_energy_forces_status": ([_vp, _vp], ctypes.c_int),
    "mp_energy_forces_noalloc": ([_vp, _P(mp_graph), _vp, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "mp_heads_create": ([_vp, _i32, _vp, _vp, _vp, _P(_vp)], ctypes.c_int),
    "mp_heads_destroy": ([_vp], ctypes.c_int),
    "mp_energy_forces_heads": ([_vp, _vp, _P(mp_graph), _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "mp_md_create": ([_vp, _i32, _f32, _f32, _f32, _vp, _P(_vp)], ctypes.c_int),
    "mp_md_set_state": ([_vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "mp_md_step": ([_vp, _i32, _vp, _vp], ctypes.c_int),
    "mp_md_use_graphs": ([_vp, _i32], ctypes.c_int),
    "mp_md_set_langevin": ([_vp, _f32, _f32], ctypes.c_int),
    "mp_md_step_nvt": ([_vp, _i32, _vp, _vp, _vp], ctypes.c_int),
    "mp_md_get_state": ([_vp, _vp, _vp, _P(_i64), _P(_i32), _P(_i32), _P(_f32), _vp], ctypes.c_int),
    "mp_md_destroy": ([_vp], ctypes.c_int),
    "mp_profile_enable": ([ctypes.c_int], ctypes.c_int),
    "mp_profile_reset": ([], ctypes.c_int),
    "mp_profile_read": ([ctypes.c_char_p, _P(ctypes.c_double), _P(_i64)], ctypes.c_int),
}
for _name, (_args, _res) in _sig.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


def _check(rc, where):
    if rc != MP_OK:
        raise MPError(rc, where)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ws(nbytes):
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device="cuda")


def cg_table(lmax):
    """Host-only: the library's real CG rows (l1, l2, l3, m1+l1, m2+l2, m3+l3, value)."""
    n = ctypes.c_int64(0)
    _check(_lib.mp_cg_table(lmax, None, 0, ctypes.byref(n)), "mp_cg_table")
    out = np.zeros((n.value, 7), np.float64)
    _check(_lib.mp_cg_table(lmax, out.ctypes.data, n.value, ctypes.byref(n)), "mp_cg_table")
    return out


def config_struct(cfg):
    return mp_model_config(cfg.n_species, cfg.channels, cfg.lmax, cfg.n_bessel, cfg.radial_hidden, cfg.heads,
                           cfg.layers, 1 if cfg.feat_bf16 else 0, cfg.cutoff)


def num_weights(cfg):
    n = ctypes.c_int64(0)
    c = config_struct(cfg)
    _check(_lib.mp_model_num_weights(ctypes.byref(c), ctypes.byref(n)), "mp_model_num_weights")
    return n.value


class Model:
    def __init__(self, cfg, weights):
        self.cfg = cfg
        w = np.ascontiguousarray(weights, np.float32)
        self._c = config_struct(cfg)
        h = ctypes.c_void_p(0)
        _check(_lib.mp_model_create(ctypes.byref(self._c), w.ctypes.data, w.size, ctypes.byref(h)),
               "mp_model_create")
        self.h = h

    @property
    def K(self):
        return (self.cfg.lmax + 1) ** 2

    def close(self):
        if self.h:
            _lib.mp_model_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Graph:
    """Sorted-slot neighbour graph on the device (owns its tensors)."""

    def __init__(self, n, L, pos, species, row_ptr, col, rev, n_edges, perm=None):
        self.n, self.L = n, float(L)
        self.pos, self.species, self.row_ptr, self.col, self.rev = pos, species, row_ptr, col, rev
        self.n_edges, self.perm = int(n_edges), perm

    def struct(self):
        return mp_graph(self.n, self.L, _ptr(self.pos), _ptr(self.species), _ptr(self.row_ptr), _ptr(self.col),
                        _ptr(self.rev), self.n_edges)


def estimate_capacity(n, L, cutoff, skin, slack=1.25):
    R = float(cutoff) + float(skin)
    rho = n / float(L) ** 3
    return int(math.ceil(slack * n * rho * 4.0 / 3.0 * math.pi * R ** 3)) + 4096


def build_neighbors(pos, species, L, cutoff, skin, capacity=None, order="hilbert"):
    """pos: cuda float32 [n,3]; species: cuda int32 [n].  Returns Graph (with perm).
    order: "hilbert" (default), "morton" or "input" (ORDERS)."""
    import torch
    n = pos.shape[0]
    dev = pos.device
    nbytes = ctypes.c_size_t(0)
    _check(_lib.mp_build_neighbors_ws(n, L, cutoff, skin, ctypes.byref(nbytes)), "mp_build_neighbors_ws")
    ws = _ws(nbytes.value)
    perm = torch.empty(n, dtype=torch.int32, device=dev)
    pos_s = torch.empty(n, 3, dtype=torch.float32, device=dev)
    sp_s = torch.empty(n, dtype=torch.int32, device=dev)
    row_ptr = torch.empty(n + 1, dtype=torch.int32, device=dev)
    cap = capacity if capacity is not None else estimate_capacity(n, L, cutoff, skin)
    for _ in range(2):
        col = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
        rev = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
        ne = ctypes.c_int64(0)
        rc = _lib.mp_build_neighbors_ordered(_ptr(pos), _ptr(species), n, L, cutoff, skin, ORDERS[order], _ptr(perm),
                                             _ptr(pos_s), _ptr(sp_s), _ptr(row_ptr), _ptr(col), _ptr(rev), cap,
                                             ctypes.byref(ne), _ptr(ws), ws.numel(), _stream())
        if rc == MP_ERR_CAPACITY and capacity is None:
            cap = ne.value
            continue
        _check(rc, "mp_build_neighbors")
        return Graph(n, L, pos_s, sp_s, row_ptr, col, rev, ne.value, perm)
    raise MPError(MP_ERR_CAPACITY, "mp_build_neighbors")


def build_neighbors_batched(pos, species, struct_ptr, cutoff, skin=0.0, capacity=None):
    """Open-boundary graph of many small structures concatenated in input order.
    pos: cuda float32 [n,3]; species: cuda int32 [n]; struct_ptr: cuda int32 [B+1].
    Returns Graph with L = 0 (open boundary) and perm = None."""
    import torch
    n, nst = pos.shape[0], struct_ptr.shape[0] - 1
    nbytes = ctypes.c_size_t(0)
    _check(_lib.mp_build_neighbors_batched_ws(n, nst, ctypes.byref(nbytes)), "mp_build_neighbors_batched_ws")
    ws = _ws(nbytes.value)
    row_ptr = torch.empty(n + 1, dtype=torch.int32, device=pos.device)
    cap = capacity if capacity is not None else 64 * n
    for _ in range(2):
        col = torch.empty(max(cap, 1), dtype=torch.int32, device=pos.device)
        rev = torch.empty(max(cap, 1), dtype=torch.int32, device=pos.device)
        ne = ctypes.c_int64(0)
        rc = _lib.mp_build_neighbors_batched(_ptr(pos), n, _ptr(struct_ptr), nst, cutoff, skin, _ptr(row_ptr),
                                             _ptr(col), _ptr(rev), cap, ctypes.byref(ne), _ptr(ws), ws.numel(),
                                             _stream())
        if rc == MP_ERR_CAPACITY and capacity is None:
            cap = ne.value
            continue
        _check(rc, "mp_build_neighbors_batched")
        return Graph(n, 0.0, pos, species, row_ptr, col, rev, ne.value, None)
    raise MPError(MP_ERR_CAPACITY, "mp_build_neighbors_batched")


def structure_energies(atom_energy, struct_ptr, out=None):
    """float64 [B] per-structure sums of the float32 atom energies (device)."""
    import torch
    nst = struct_ptr.shape[0] - 1
    out = torch.empty(nst, dtype=torch.float64, device=atom_energy.device) if out is None else out
    _check(_lib.mp_structure_energies(_ptr(atom_energy), _ptr(struct_ptr), nst, _ptr(out), _stream()),
           "mp_structure_energies")
    return out


def feat_dtype(model):
    import torch
    return torch.int16 if model.cfg.feat_bf16 else torch.float32


def embed(model, g):
    import torch
    h = torch.empty(g.n, model.K, model.cfg.channels, dtype=feat_dtype(model), device="cuda")
    gs = g.struct()
    _check(_lib.mp_embed(model.h, ctypes.byref(gs), _ptr(h), _stream()), "mp_embed")
    return h


def layer_forward(model, layer, g, h_in):
    import torch
    nbytes = ctypes.c_size_t(0)
    _check(_lib.mp_layer_forward_ws(model.h, g.n, max(g.n_edges, 1), ctypes.byref(nbytes)), "mp_layer_forward_ws")
    ws = _ws(nbytes.value)
    h_out = torch.empty_like(h_in)
    gs = g.struct()
    _check(_lib.mp_layer_forward(model.h, layer, ctypes.byref(gs), _ptr(h_in), _ptr(h_out), _ptr(ws), ws.numel(),
                                 _stream()), "mp_layer_forward")
    return h_out


class EnergyForces:
    """Reusable workspace for repeated mp_energy_forces calls on one graph size."""

    def __init__(self, model, n, capacity):
        import torch
        self.model = model
        nbytes = ctypes.c_size_t(0)
        _check(_lib.mp_energy_forces_ws(model.h, n, max(int(capacity), 1), ctypes.byref(nbytes)),
               "mp_energy_forces_ws")
        self.nbytes = nbytes.value
        self.ws = _ws(nbytes.value)
        self.energy = torch.zeros(1, dtype=torch.float64, device="cuda")
        self.n, self.capacity = n, capacity

    def __call__(self, g, perm=None, forces=None, atom_energy=None, stream=None, check=True):
        """Enqueue mp_energy_forces; check: then wait for it and raise MPError (MP_ERR_NUMERIC)
        if the energy or a force is non-finite (mp_energy_forces_status)."""
        import torch
        if g.n != self.n or g.n_edges > self.capacity:
            raise ValueError("graph does not fit this workspace")
        if forces is None:
            forces = torch.empty(g.n, 3, dtype=torch.float32, device="cuda")
        gs = g.struct()
        st = ctypes.c_void_p(stream) if stream is not None else _stream()
        _check(_lib.mp_energy_forces(self.model.h, ctypes.byref(gs), _ptr(perm), _ptr(self.energy), _ptr(forces),
                                     _ptr(atom_energy), _ptr(self.ws), self.ws.numel(), st), "mp_energy_forces")
        if check:
            self.status(st)
        return self.energy, forces

    def status(self, stream=None):
        st = ctypes.c_void_p(stream) if isinstance(stream, int) else (stream or _stream())
        _check(_lib.mp_energy_forces_status(_ptr(self.ws), st), "mp_energy_forces_status")


def energy_forces_noalloc(model, g, energy, forces, perm=None, atom_energy=None, nonfinite=None):
    """mp_energy_forces_noalloc into caller tensors (energy float64 [1], forces float32 [n][3],
    atom_energy float32 [n] or None, nonfinite int32 [1] or None); enqueues only."""
    gs = g.struct()
    _check(_lib.mp_energy_forces_noalloc(model.h, ctypes.byref(gs), _ptr(perm), _ptr(energy), _ptr(forces),
                                         _ptr(atom_energy), _ptr(nonfinite), _stream()), "mp_energy_forces_noalloc")


def energy_forces(model, g, perm=None, atom_energy=None):
    ef = EnergyForces(model, g.n, max(g.n_edges, 1))
    E, F = ef(g, perm=perm, atom_energy=atom_energy)
    return float(E.item()), F


class Heads:
    """R readout heads on one model's encoder (mp_heads_create): wr [R][C][C] (out, in),
    wout [R][C], lam [R], host arrays."""

    def __init__(self, model, wr, wout, lam):
        wr = np.ascontiguousarray(wr, np.float32)
        wout = np.ascontiguousarray(wout, np.float32)
        lam = np.ascontiguousarray(lam, np.float32)
        R, C = lam.size, model.cfg.channels
        if wr.shape != (R, C, C) or wout.shape != (R, C):
            raise ValueError(f"heads: want wr [{R}][{C}][{C}] and wout [{R}][{C}]")
        h = ctypes.c_void_p(0)
        _check(_lib.mp_heads_create(model.h, R, wr.ctypes.data, wout.ctypes.data, lam.ctypes.data, ctypes.byref(h)),
               "mp_heads_create")
        self.h, self.R, self.model = h, R, model

    def close(self):
        if self.h:
            _lib.mp_heads_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def energy_forces_heads(model, heads, g, perm=None, ws=None):
    """mp_energy_forces_heads: returns (head energies float64 [R] (device), E = sum_k lam_k E_k
    (float), forces [n][3], per-head atom energies [R][n] (device, slot order))."""
    import torch
    if ws is None:
        nbytes = ctypes.c_size_t(0)
        _check(_lib.mp_energy_forces_ws(model.h, g.n, max(g.n_edges, 1), ctypes.byref(nbytes)),
               "mp_energy_forces_ws")
        ws = _ws(nbytes.value)
    e_heads = torch.zeros(heads.R, dtype=torch.float64, device="cuda")
    energy = torch.zeros(1, dtype=torch.float64, device="cuda")
    forces = torch.empty(g.n, 3, dtype=torch.float32, device="cuda")
    e_atoms = torch.empty(heads.R, g.n, dtype=torch.float32, device="cuda")
    gs = g.struct()
    _check(_lib.mp_energy_forces_heads(model.h, heads.h, ctypes.byref(gs), _ptr(perm), _ptr(e_heads), _ptr(energy),
                                       _ptr(forces), _ptr(e_atoms), _ptr(ws), ws.numel(), _stream()),
           "mp_energy_forces_heads")
    _check(_lib.mp_energy_forces_status(_ptr(ws), _stream()), "mp_energy_forces_status")
    return e_heads, float(energy.item()), forces, e_atoms


class MD:
    """Velocity-Verlet NVE handle (mp_md_*).  masses: per species, amu."""

    def __init__(self, model, n, L, skin, dt_fs, masses):
        self.model, self.n = model, n
        m = np.ascontiguousarray(masses, np.float32)
        h = ctypes.c_void_p(0)
        _check(_lib.mp_md_create(model.h, n, L, skin, dt_fs, m.ctypes.data, ctypes.byref(h)), "mp_md_create")
        self.h = h

    def set_state(self, pos, vel, species):
        _check(_lib.mp_md_set_state(self.h, _ptr(pos), _ptr(vel), _ptr(species), _stream()), "mp_md_set_state")

    def use_graphs(self, enable=True):
        """replay captured step graphs (default) or enqueue each step's kernels"""
        _check(_lib.mp_md_use_graphs(self.h, 1 if enable else 0), "mp_md_use_graphs")

    def set_langevin(self, temperature_K, gamma_per_ps):
        """BAOAB Langevin thermostat (gamma > 0), or back to NVE (gamma = 0)"""
        _check(_lib.mp_md_set_langevin(self.h, float(temperature_K), float(gamma_per_ps)), "mp_md_set_langevin")

    def step_nvt(self, noise, e_log=True):
        """Advance len(noise) Langevin steps; noise: cuda float32 [n_steps][n][3] standard normals
        in input-atom order.  Returns numpy [n_steps][2] (kinetic, potential) or None."""
        import torch
        n_steps = noise.shape[0]
        assert noise.dtype == torch.float32 and noise.is_cuda and noise.is_contiguous()
        assert tuple(noise.shape[1:]) == (self.n, 3)
        log = torch.zeros(max(n_steps, 1), 2, dtype=torch.float64, device="cuda") if e_log else None
        _check(_lib.mp_md_step_nvt(self.h, n_steps, _ptr(noise), _ptr(log), _stream()), "mp_md_step_nvt")
        return log[:n_steps].cpu().numpy() if e_log else None

    def step(self, n_steps, e_log=True):
        """Advance n_steps; returns numpy [n_steps][2] (kinetic, potential) in eV, or None."""
        import torch
        log = torch.zeros(max(n_steps, 1), 2, dtype=torch.float64, device="cuda") if e_log else None
        _check(_lib.mp_md_step(self.h, n_steps, _ptr(log), _stream()), "mp_md_step")
        return log[:n_steps].cpu().numpy() if e_log else None

    def state(self):
        import torch
        pos = torch.empty(self.n, 3, dtype=torch.float32, device="cuda")
        vel = torch.empty(self.n, 3, dtype=torch.float32, device="cuda")
        step, nreb, ncap, dmin = ctypes.c_int64(0), ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_float(0)
        _check(_lib.mp_md_get_state(self.h, _ptr(pos), _ptr(vel), ctypes.byref(step), ctypes.byref(nreb),
                                    ctypes.byref(ncap), ctypes.byref(dmin), _stream()), "mp_md_get_state")
        return {"pos": pos.cpu().numpy(), "vel": vel.cpu().numpy(), "step": step.value, "n_rebuilds": nreb.value,
                "n_captures": ncap.value, "min_pair": dmin.value}

    def close(self):
        if self.h:
            _lib.mp_md_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def profile_enable(on=True):
    _check(_lib.mp_profile_enable(1 if on else 0), "mp_profile_enable")


def profile_reset():
    _check(_lib.mp_profile_reset(), "mp_profile_reset")


def profile_read(name):
    """(total_ms, launches) for kernel `name` since the last reset."""
    ms, n = ctypes.c_double(0), ctypes.c_int64(0)
    _check(_lib.mp_profile_read(name.encode(), ctypes.byref(ms), ctypes.byref(n)), "mp_profile_read")
    return ms.value, n.value


def bf16_to_f32(t):
    """int16 bit patterns of bfloat16 -> float32 tensor."""
    import torch
    return (t.to(torch.int32) << 16).view(torch.float32)
