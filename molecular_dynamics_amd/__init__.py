"""MI355X-native equivariant message-passing attention energy/force path.

``molecular_dynamics_amd.mdmp`` is the thin ctypes binding over the C-ABI
library ``libmdmp.so`` (HIP kernels for gfx950); importing it fails loudly when
the library is missing.  ``molecular_dynamics_amd.inputs`` holds the seeded
synthetic boxes and weights.
"""
