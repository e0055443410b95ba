"""MI355X (gfx950) 3D star stencil and acoustic wave step.

The compute path is ``libstencil3d.so``: hand-written HIP kernels behind a
C ABI (``include/stencil3d.h``).  ``acoustic_wave_propagation_amd.binding``
marshals torch device tensors into that ABI; importing this package does not
load the library, so the input generators (``workloads``) and the
byte-accounting helpers (``traffic``) work on machines without a GPU.
"""

__all__ = ["binding", "workloads", "traffic"]
