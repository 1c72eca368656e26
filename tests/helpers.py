"""Shared test helpers: workloads, oracle runs, tolerance checks."""
import functools

import numpy as np


@functools.lru_cache(maxsize=None)
def workload(name):
    from molecular_dynamics_amd import inputs
    return inputs.workload(name)


def to_dev(box):
    import torch
    pos = torch.tensor(box.pos, device="cuda")
    sp = torch.tensor(box.species, device="cuda")
    return pos, sp


def force_error(F, Fref):
    """max atom-wise |dF| / max atom-wise |F_ref|."""
    return float(np.linalg.norm(F - Fref, axis=1).max() / np.linalg.norm(Fref, axis=1).max())


def energy_error(E, Eref, e_atoms_ref):
    return abs(E - Eref) / float(np.abs(e_atoms_ref).sum())
