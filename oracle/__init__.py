"""CPU oracle for the q4_K x q8 quantized matmul (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path never does.
"""
from .oracle import (blockdots, build, f16_bits, f16_to_f64, load, out_f64,  # noqa: F401
                     q4k_repack, q4k_unpack, q8_tiles, q6k_dots, q6k_out_f64, q6k_unpack, quantize, quantize_silu_mul, silu_mul,
                     set_threads, get_threads)
