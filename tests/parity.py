"""Float comparison rules used by the GPU parity tests (defined in oracle/compare.py)."""
from oracle.compare import bf16_to_f64, bf16_ulp, check_float, f64_to_bf16_val  # noqa: F401
