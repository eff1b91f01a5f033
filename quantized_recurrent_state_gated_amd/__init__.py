"""Quantized recurrent-state decode step for MI355X (gfx950).

The fused gated delta-rule decode step over a per-request pool of 4/6/8-bit
recurrent states with FP16 pivot heads, as hand-written HIP kernels behind a
C-ABI library (``libsq.so``, declared in ``include/sq.h``).

``quantized_recurrent_state_gated_amd.sq`` is the Python binding (argument
marshalling only); ``quantized_recurrent_state_gated_amd.inputs`` draws the
seeded synthetic workloads.  Importing this package loads nothing; importing
``.sq`` loads the library and fails loudly if it has not been built.
"""
