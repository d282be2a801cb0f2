"""CPU oracle of the dropless MoE expert-FFN layer (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``ragged_grouped_gemm_amd``) and neither imports the other; the seeded input
generator ``synth`` is the only module both sides use.

``oracle.moe``: routing, permutation, FC1 weight repack, GLU activations,
grouped GEMMs, combine and the whole forward / backward chain in float64.
``oracle.mx``: the OCP MXFP8 codec (E4M3 elements, E8M0 block scales).
"""
from . import moe, mx  # noqa: F401
