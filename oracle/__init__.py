"""CPU oracle for paged-KV attention: plain, slow, fp64.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package's smoke
entry point and by the benchmark's CPU-baseline leg, never by the library or
its binding.  It shares no code with the HIP path.
"""
from .paged_attention import (  # noqa: F401
    PAGE_SIZE, DTYPES, SCALED, PagedCache, bf16_bits_to_f64, e4m3_bits_to_f64, f32_to_bf16_bits,
    f32_to_e4m3_bits, f32_to_f16, quantize_fp8,
    gather_sequence, max_abs_err, quantize_int8, ref_append, ref_append_rope, ref_decode,
    ref_prefill_chunk, ref_rope_q, rope_f64, storage_from_f32, upcast,
)
