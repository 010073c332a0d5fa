"""CPU oracle for paged-KV attention prefill.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the library.  See attention.py and
sampling.py.
"""
from .attention import (NEG_INF, allowed_mask, append_paged_kv, attention,
                        attention_bruteforce, attention_rows, custom_mask_rows,
                        decode_e4m3, gather_request_kv, kv_lengths, merge_many, merge_states,
                        soft_cap)
from .sampling import chain_speculative_sampling, inverse_cdf

__all__ = ["NEG_INF", "allowed_mask", "append_paged_kv", "attention", "attention_bruteforce",
           "attention_rows", "custom_mask_rows", "gather_request_kv", "kv_lengths",
           "merge_many", "merge_states", "soft_cap", "decode_e4m3", "chain_speculative_sampling", "inverse_cdf"]
