"""CPU oracle for the equivariant message-passing attention potential.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
CPU statement of what the GPU path computes, written from the method's
description in "Ab Initio Accuracy Beyond the Cutoff: Distributed
Message-Passing Equivariant Attention at Tens-of-Millions-of-Atom Scale"
(Abstract) and the design notes of "Unlocking Tensor Core Performance: GPU
Acceleration for Machine Learning Interatomic Potentials".  It shares no code
with the HIP library and never calls it.  Only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
it; the product path must never route through it.

Precision: float64 throughout, starting from the same float32 positions and
weights the GPU path receives.

Modules
  hilbert    -- space-filling-curve keys (Skilling's transpose algorithm)
  neighbors  -- wrap, Hilbert sort, skin-padded radius graph (sorted CSR), reverse edges
  basis      -- real spherical harmonics, Bessel radial basis, polynomial envelope
  cg         -- real Clebsch-Gordan intertwiners (null-space construction)
  model      -- the attention layer stack, energy, forces by autograd
  md         -- velocity-Verlet NVE stepping with skin-triggered rebuilds
Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
brute force, symmetry or calculus; see each test's docstring.
"""
