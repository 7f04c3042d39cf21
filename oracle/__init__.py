"""CPU oracle for exact attention (numpy float64).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the GPU product path.
"""
from .attention import (attention_backward, attention_backward_head,
                        attention_decode, attention_decode_fp8, attention_prefill,
                        attention_prefill_fp8, attention_prefill_paged_fp8,
                        attention_prefill_varlen_fp8,
                        attention_prefill_paged, attention_prefill_varlen,
                        attention_probabilities,
                        attention_rows, brute_force_attention, e4m3_value, gather_paged,
                        merge_partials, online_attention, softmax_rows)

__all__ = ["attention_backward", "attention_backward_head",
           "attention_decode", "attention_decode_fp8", "attention_prefill",
           "attention_prefill_fp8", "attention_prefill_paged_fp8",
           "attention_prefill_varlen_fp8",
           "attention_prefill_paged", "attention_prefill_varlen", "attention_probabilities",
           "attention_rows",
           "brute_force_attention", "e4m3_value", "gather_paged", "merge_partials",
           "online_attention", "softmax_rows"]
