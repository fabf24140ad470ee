"""MI355X-native BitLinear forward path with I2_S ternary weights.

``ternary_weight_amd.bitlinear`` binds the C-ABI library ``libbitlinear.so``
(hand-written HIP for gfx950); ``ternary_weight_amd.inputs`` generates the
seeded synthetic workloads.  Importing this package loads nothing; importing
``ternary_weight_amd.bitlinear`` raises if the library has not been built.
"""
