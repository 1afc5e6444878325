"""CPU float64 oracle (test infrastructure only; never on the product path)."""
from .attention import (BF16, FP16, admissible_mask, attention_bwd_dq_rows_ref,
                        attention_bwd_ref, attention_ref, attention_rows_ref, decode_multi_ref,
                        decode_paged_ref, decode_ref, lse_ref, merge_ref, partial_ref, probs_ref,
                        varlen_ref, widen)

__all__ = ["BF16", "FP16", "admissible_mask", "attention_bwd_dq_rows_ref", "attention_bwd_ref",
           "attention_ref", "attention_rows_ref", "decode_multi_ref", "decode_paged_ref",
           "decode_ref", "lse_ref", "merge_ref", "partial_ref", "probs_ref", "varlen_ref", "widen"]
