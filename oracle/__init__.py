"""Plain fp64 CPU oracle for the EQ-Linear layer (cyclic groups C_T and
dihedral groups D_n) and for the p4 group convolution built from it.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP path (no kernels, headers,
helpers, tables or constants) and imports nothing from it.

What it computes, and where each piece is defined, is documented per function in
``oracle/eqlinear_oracle.py`` and ``oracle/eqconv_oracle.py``.  Every function has pins in ``tests/`` that tie
it to the definition on the pages and to mathematics (brute force, closed
forms, special cases that reduce to library routines, invariants, finite
differences); none of it is "parity unpinned".
"""
from .eqlinear_oracle import (  # noqa: F401
    GROUPS,
    dihedral_multiply,
    dihedral_inverse,
    tap_table,
    unroll_group,
    unroll_block_circulant,
    forward,
    gelu,
    gelu_tanh,
    forward_act,
    backward_input,
    backward_weight,
    mac_counts,
    param_counts,
)
from .eqconv_oracle import (  # noqa: F401
    rotate_offset,
    tap_matrix,
    conv_forward,
    conv_forward_act,
    conv_backward_input,
    conv_backward_weight,
    conv_mac_counts,
    conv_param_counts,
)
