"""CPU fp64 oracle (test infrastructure only; never imported by the library)."""
from .attention import (cache_write_ref, decode_partials_ref, decode_ref, gather_sequence, lse_merge_ref,
                        paged_attention_ref)

__all__ = ["cache_write_ref", "decode_partials_ref", "decode_ref", "gather_sequence", "lse_merge_ref",
           "paged_attention_ref"]
