"""Seeded synthetic inputs: atom boxes, model weights, initial velocities.

This module is shared by the CPU oracle and the GPU path, so it holds none of
the potential's arithmetic: it only draws random numbers and lays them out.

The boxes stand in for the workloads of "Ab Initio Accuracy Beyond the
Cutoff: Distributed Message-Passing Equivariant Attention at
Tens-of-Millions-of-Atom Scale" (Abstract: a salt solution and a virus capsid,
neither of which is available here).  Salt boxes use rigid three-site waters
plus Na/Cl ions; the heterogeneous box puts a dense spherical shell of mixed
species in a dilute solvent, which mimics a capsid's density contrast.

Every box is built by random sequential addition (RSA) with a 1.0 A minimum
separation (minimum image) between atoms of different molecules.  Randomness
comes from one integer seed per workload, split with
``numpy.random.SeedSequence(seed).spawn(3)`` into positions, species and
weights.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))

# ---------------------------------------------------------------------------
# model configuration and weight blob layout
# ---------------------------------------------------------------------------


@dataclass
class ModelConfig:
    n_species: int
    channels: int
    lmax: int
    n_bessel: int
    heads: int
    layers: int
    cutoff: float
    radial_hidden: int = 64
    feat_bf16: bool = False

    @property
    def n_paths(self) -> int:
        # number of (l1, l2, l3) triples with 0 <= l <= lmax obeying the
        # triangle rule |l1 - l2| <= l3 <= l1 + l2 (a shape, not arithmetic)
        return sum(1 for a in range(self.lmax + 1) for b in range(self.lmax + 1)
                   for c in range(self.lmax + 1) if abs(a - b) <= c <= a + b)


def weight_layout(cfg: ModelConfig):
    """Blob layout: list of (name, rows, cols), row-major [out][in], in order."""
    C, H = cfg.channels, cfg.radial_hidden
    out = [("emb", cfg.n_species, C)]
    for t in range(cfg.layers):
        out.append((f"l{t}.w1", H, cfg.n_bessel))
        out.append((f"l{t}.w2", cfg.n_paths * C, H))
        out.append((f"l{t}.wq", C, C))
        for l in range(cfg.lmax + 1):
            out.append((f"l{t}.wv{l}", C, C))
        for l in range(cfg.lmax + 1):
            out.append((f"l{t}.wo{l}", C, C))
        out.append((f"l{t}.wg", cfg.lmax * C, C))
    out.append(("wr", C, C))
    out.append(("wout", 1, C))
    return out


def make_weights(cfg: ModelConfig, seed_seq) -> np.ndarray:
    """N(0, 1/fan_in) weights in blob order, fp32.  fan_in of the embedding is 1."""
    rng = np.random.default_rng(seed_seq)
    parts = []
    for name, r, c in weight_layout(cfg):
        fan_in = 1 if name == "emb" else c
        parts.append((rng.standard_normal((r, c)) / math.sqrt(fan_in)).astype(np.float32).ravel())
    return np.concatenate(parts)


def split_weights(cfg: ModelConfig, flat: np.ndarray) -> dict:
    """Views of the blob by name (layout bookkeeping only)."""
    out, off = {}, 0
    for name, r, c in weight_layout(cfg):
        out[name] = flat[off:off + r * c].reshape(r, c)
        off += r * c
    assert off == flat.size, (off, flat.size)
    return out


# ---------------------------------------------------------------------------
# random sequential addition (C helper, built with gcc on first use)
# ---------------------------------------------------------------------------

_RSA_SO = os.path.join(_HERE, "_rsa.so")
_rsa_lib = None


def build_rsa(force: bool = False) -> str:
    src = os.path.join(_HERE, "_rsa.c")
    if force or not os.path.exists(_RSA_SO) or os.path.getmtime(_RSA_SO) < os.path.getmtime(src):
        tmp = _RSA_SO + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-shared", "-fPIC", "-o", tmp, src, "-lm"])
        os.replace(tmp, _RSA_SO)
    return _RSA_SO


def _rsa():
    global _rsa_lib
    if _rsa_lib is None:
        lib = ctypes.CDLL(build_rsa())
        lib.rsa_create.restype = ctypes.c_void_p
        lib.rsa_create.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_int64]
        lib.rsa_destroy.argtypes = [ctypes.c_void_p]
        lib.rsa_add.restype = ctypes.c_int64
        lib.rsa_add.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64)]
        _rsa_lib = lib
    return _rsa_lib


class _Packer:
    def __init__(self, L, cap, min_sep=1.0):
        self.lib = _rsa()
        self.L = float(L)
        self.h = self.lib.rsa_create(self.L, float(min_sep), int(cap))

    def add(self, draw, n_target, atoms_per, batch=65536, max_batches=10000):
        """draw(k) -> candidate molecules [k][atoms_per][3]; returns [n_target][atoms_per][3]."""
        out = np.zeros((n_target, atoms_per, 3), np.float64)
        n_acc = ctypes.c_int64(0)
        for _ in range(max_batches):
            if n_acc.value >= n_target:
                break
            cand = np.ascontiguousarray(draw(batch), dtype=np.float64)
            rc = self.lib.rsa_add(self.h, cand.ctypes.data, cand.shape[0], atoms_per, n_target,
                                  out.ctypes.data, ctypes.byref(n_acc))
            if rc < 0:
                raise RuntimeError(f"RSA packing failed ({rc})")
        if n_acc.value < n_target:
            raise RuntimeError("RSA did not reach the target count")
        return out

    def close(self):
        if self.h:
            self.lib.rsa_destroy(self.h)
            self.h = None


# ---------------------------------------------------------------------------
# boxes
# ---------------------------------------------------------------------------

WATER_OH = 0.9572          # A, rigid three-site water geometry
WATER_HOH = 104.52         # degrees
MOLAR = 6.02214076e-4      # 1 mol/L in molecules per A^3
SPECIES_SALT = {"O": 0, "H": 1, "Na": 2, "Cl": 3}
MASSES_SALT = np.array([15.999, 1.008, 22.990, 35.45], np.float32)   # amu, by species id


@dataclass
class Box:
    pos: np.ndarray          # [N,3] float32, inside [0, L)
    species: np.ndarray      # [N] int32
    L: float                 # float32-representable side
    n_species: int
    meta: dict = field(default_factory=dict)

    @property
    def n(self):
        return self.pos.shape[0]


def _uniform(rng, L):
    return lambda k: rng.random((k, 1, 3)) * L


def box_uniform(n, L, n_species, seed, species_ratio=None):
    ss_pos, ss_sp, _ = np.random.SeedSequence(seed).spawn(3)
    rng = np.random.default_rng(ss_pos)
    pk = _Packer(L, n)
    try:
        pos = pk.add(_uniform(rng, L), n, 1, batch=max(1024, n // 4)).reshape(n, 3)
    finally:
        pk.close()
    rs = np.random.default_rng(ss_sp)
    if species_ratio is None:
        sp = rs.integers(0, n_species, size=n)
    else:
        w = np.asarray(species_ratio, np.float64)
        counts = np.floor(n * w / w.sum()).astype(np.int64)
        counts[0] += n - counts.sum()
        sp = rs.permutation(np.repeat(np.arange(n_species), counts))
    return Box(_f32_box(pos, L), sp.astype(np.int32), float(np.float32(L)), n_species)


def _f32_box(pos, L):
    p = pos.astype(np.float32)
    Lf = np.float32(L)
    p[p >= Lf] = 0.0
    p[p < 0] = 0.0
    return p


def _random_rotations(rng, k):
    q = rng.standard_normal((k, 4))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    w, x, y, z = q.T
    R = np.empty((k, 3, 3))
    R[:, 0, 0] = 1 - 2 * (y * y + z * z); R[:, 0, 1] = 2 * (x * y - z * w); R[:, 0, 2] = 2 * (x * z + y * w)
    R[:, 1, 0] = 2 * (x * y + z * w); R[:, 1, 1] = 1 - 2 * (x * x + z * z); R[:, 1, 2] = 2 * (y * z - x * w)
    R[:, 2, 0] = 2 * (x * z - y * w); R[:, 2, 1] = 2 * (y * z + x * w); R[:, 2, 2] = 1 - 2 * (x * x + y * y)
    return R


def _water_template():
    th = math.radians(WATER_HOH) / 2
    return np.array([[0.0, 0.0, 0.0],
                     [WATER_OH * math.sin(th), 0.0, WATER_OH * math.cos(th)],
                     [-WATER_OH * math.sin(th), 0.0, WATER_OH * math.cos(th)]])


def salt_counts(n):
    """(n_pair, n_water, L): ions at 1 mol/L, water atoms at exactly 0.1 /A^3."""
    target = n * MOLAR / (0.1 + 2 * MOLAR)
    best = None
    for k in range(max(0, int(target) - 6), int(target) + 7):
        if (n - 2 * k) % 3 == 0 and (best is None or abs(k - target) < abs(best - target)):
            best = k
    n_water = (n - 2 * best) // 3
    L = float(np.float32((10.0 * 3 * n_water) ** (1.0 / 3.0)))
    return best, n_water, L


def box_salt(n, seed):
    n_pair, n_water, L = salt_counts(n)
    ss_pos, _, _ = np.random.SeedSequence(seed).spawn(3)
    rng = np.random.default_rng(ss_pos)
    pk = _Packer(L, n)
    try:
        ions = pk.add(_uniform(rng, L), 2 * n_pair, 1, batch=4096).reshape(-1, 3)
        tmpl = _water_template()

        def draw_water(k):
            R = _random_rotations(rng, k)
            c = rng.random((k, 3)) * L
            return c[:, None, :] + np.einsum("kij,aj->kai", R, tmpl)

        waters = pk.add(draw_water, n_water, 3, batch=65536).reshape(-1, 3)
    finally:
        pk.close()
    pos = np.concatenate([ions, waters])
    sp = np.concatenate([np.full(n_pair, SPECIES_SALT["Na"]), np.full(n_pair, SPECIES_SALT["Cl"]),
                         np.tile([SPECIES_SALT["O"], SPECIES_SALT["H"], SPECIES_SALT["H"]], n_water)])
    return Box(_f32_box(pos, L), sp.astype(np.int32), L, 4,
               meta={"n_pair": n_pair, "n_water": n_water})


def shell_box_side(n, rho_shell=0.12, rho_solv=0.1, r_in=0.3, r_out=0.4):
    v_shell_frac = 4.0 / 3.0 * math.pi * (r_out ** 3 - r_in ** 3)
    return float(np.float32((n / (rho_solv + (rho_shell - rho_solv) * v_shell_frac)) ** (1.0 / 3.0)))


def box_shell(n, seed, n_species=5, rho_shell=0.12, rho_solv=0.1):
    """Dense spherical shell (radii 0.3L..0.4L about the centre) in dilute solvent."""
    L = shell_box_side(n, rho_shell, rho_solv)
    r_in, r_out = 0.3 * L, 0.4 * L
    n_shell = int(round(rho_shell * 4.0 / 3.0 * math.pi * (r_out ** 3 - r_in ** 3)))
    n_solv = n - n_shell
    ss_pos, ss_sp, _ = np.random.SeedSequence(seed).spawn(3)
    rng = np.random.default_rng(ss_pos)
    ctr = np.full(3, L / 2)

    def draw(inside):
        def f(k):
            out = []
            got = 0
            while got < k:
                c = rng.random((k, 3)) * L
                r = np.linalg.norm(c - ctr, axis=1)
                m = (r >= r_in) & (r <= r_out)
                c = c[m if inside else ~m]
                out.append(c)
                got += c.shape[0]
            return np.concatenate(out)[:k, None, :]
        return f

    pk = _Packer(L, n)
    try:
        shell = pk.add(draw(True), n_shell, 1, batch=65536).reshape(-1, 3)
        solv = pk.add(draw(False), n_solv, 1, batch=65536).reshape(-1, 3)
    finally:
        pk.close()
    rs = np.random.default_rng(ss_sp)
    sp = np.concatenate([rs.integers(0, n_species, size=n_shell), np.zeros(n_solv, np.int64)])
    return Box(_f32_box(np.concatenate([shell, solv]), L), sp.astype(np.int32), L, n_species,
               meta={"n_shell": n_shell, "n_solvent": n_solv})


def maxwell_boltzmann(masses_amu, temperature_k, seed):
    """Initial velocities (A/fs): N(0, kB*T/m) per component, centre-of-mass motion removed."""
    kb_ev = 8.617333262e-5
    ev_per_amu_a2_fs2 = 103.642696    # 1 amu*(A/fs)^2 in eV
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(3)[2])
    m = np.asarray(masses_amu, np.float64)
    sig = np.sqrt(kb_ev * temperature_k / (m * ev_per_amu_a2_fs2))
    v = rng.standard_normal((m.size, 3)) * sig[:, None]
    v -= (m[:, None] * v).sum(0) / m.sum()
    return v.astype(np.float32)


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

SEEDS = {"tiny64": 1101, "dense4k": 1102, "salt262k": 1103, "shell1m": 1104, "salt131k_md": 1105,
         "salt4k_md": 1106, "mol16k": 1107, "salt512_md": 1108}


def batch_molecules(n_struct, n_min, n_max, seed, rho=0.1, min_sep=1.0, n_species=4):
    """A batch of small open structures (molecule-like clusters): structure b has n_b atoms, n_b uniform
    in [n_min, n_max], placed by random sequential addition (min_sep apart) in a ball of radius
    (3 n_b / (4 pi rho))^(1/3) about the origin; species uniform.  Returns (pos float32 [N,3],
    species int32 [N], struct_ptr int32 [B+1]), structures concatenated."""
    ss_pos, ss_sp, _ = np.random.SeedSequence(seed).spawn(3)
    rng = np.random.default_rng(ss_pos)
    sizes = rng.integers(n_min, n_max + 1, n_struct)
    radius = (3.0 * sizes / (4.0 * np.pi * rho)) ** (1.0 / 3.0)
    x = np.full((n_struct, n_max, 3), np.nan)
    for k in range(n_max):
        todo = np.nonzero(sizes > k)[0]
        while todo.size:
            c = rng.random((todo.size, 3)) * 2.0 - 1.0
            ok = (c * c).sum(1) <= 1.0
            c = c * radius[todo, None]
            if k:
                d = x[todo, :k, :] - c[:, None, :]
                ok &= np.nanmin((d * d).sum(2), axis=1) >= min_sep * min_sep
            x[todo[ok], k] = c[ok]
            todo = todo[~ok]
    pos = np.concatenate([x[b, :sizes[b]] for b in range(n_struct)]).astype(np.float32)
    sp = np.random.default_rng(ss_sp).integers(0, n_species, pos.shape[0]).astype(np.int32)
    sptr = np.zeros(n_struct + 1, np.int32)
    sptr[1:] = np.cumsum(sizes)
    return pos, sp, sptr


def molecule_batch(name="mol16k"):
    """16,384 structures of 8-32 atoms with the 1M-atom box's model (C = 128, lmax 2, 4 layers,
    4 heads, r_c 5 A, bf16 features; 4 species): the batched-throughput workload (structures/s)."""
    seed = SEEDS[name]
    pos, sp, sptr = batch_molecules(16384, 8, 32, seed)
    cfg = ModelConfig(n_species=4, channels=128, lmax=2, n_bessel=8, heads=4, layers=4, cutoff=5.0, feat_bf16=True)
    w = make_weights(cfg, np.random.SeedSequence(seed).spawn(3)[2])
    return pos, sp, sptr, cfg, w


@dataclass
class Workload:
    name: str
    box: Box
    model: ModelConfig
    skin: float
    weights: np.ndarray
    extra: dict = field(default_factory=dict)


def workload(name: str) -> Workload:
    seed = SEEDS[name]
    _, _, ss_w = np.random.SeedSequence(seed).spawn(3)
    if name == "tiny64":
        box = box_uniform(64, 12.0, 2, seed)
        cfg = ModelConfig(n_species=2, channels=16, lmax=1, n_bessel=8, heads=2, layers=1, cutoff=5.0)
        skin = 0.0
    elif name == "dense4k":
        box = box_uniform(4096, (4096 / 0.1) ** (1 / 3), 3, seed, species_ratio=(2, 1, 1))
        cfg = ModelConfig(n_species=3, channels=64, lmax=2, n_bessel=8, heads=4, layers=2, cutoff=5.0)
        skin = 0.0
    elif name == "salt262k":
        box = box_salt(262144, seed)
        cfg = ModelConfig(n_species=4, channels=128, lmax=2, n_bessel=8, heads=4, layers=4, cutoff=6.0,
                          feat_bf16=True)
        skin = 1.0
    elif name == "shell1m":
        box = box_shell(1 << 20, seed)
        cfg = ModelConfig(n_species=5, channels=128, lmax=2, n_bessel=8, heads=4, layers=4, cutoff=5.0,
                          feat_bf16=True)
        skin = 1.0
    elif name in ("salt131k_md", "salt4k_md", "salt512_md"):
        box = box_salt({"salt131k_md": 131072, "salt4k_md": 4096, "salt512_md": 512}[name], seed)
        cfg = ModelConfig(n_species=4, channels=128, lmax=2, n_bessel=8, heads=4, layers=4, cutoff=6.0)
        skin = 1.0
    else:
        raise KeyError(name)
    w = make_weights(cfg, ss_w)
    extra = {}
    if name.endswith("_md"):
        masses = MASSES_SALT[box.species]
        extra = {"masses": MASSES_SALT.copy(), "vel": maxwell_boltzmann(masses, 300.0, seed),
                 "dt_fs": 0.5, "steps": 2000}
    return Workload(name, box, cfg, skin, w, extra)
