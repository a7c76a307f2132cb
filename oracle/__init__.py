"""fp64 CPU oracle for paged decode (test infrastructure; never used by the product path)."""
from .pa_oracle import (FP8_E4M3_TABLE, attend, bf16_bits_to_f64, decode, decode_batch,  # noqa: F401
                        fp8_e4m3_value, gather, kv_cache_bytes, kv_unique_bytes, lse_merge,
                        paged_decode, partial_state)
