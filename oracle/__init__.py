"""CPU oracle for fused scaled-dot-product attention (test infrastructure).

Only the tests, the smoke entry point and the benchmark's CPU-baseline leg may
import this package; the HIP path never does, and this package never imports
the HIP path.
"""

from .oracle import bf16_bits_to_f64, dequant_blocks, alibi_slopes, attend_rows, prefill, decode_paged, decode_gathered, mla_tail  # noqa: F401
