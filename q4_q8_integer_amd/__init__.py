"""q4_K x q8 quantized matmul (MMQ) for MI355X (gfx950).

The HIP library is loaded on first use by ``q4_q8_integer_amd.binding``;
importing the package itself loads nothing.
"""
