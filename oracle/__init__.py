"""CPU oracle for the exact-attention forward pass.

Test infrastructure only: imported by tests/, the smoke check and the benchmark's
CPU-baseline leg, never by the library or its Python binding.
"""

from .attention import attention_bruteforce, attention_bwd_ref, attention_ref, kv_head_of
from .varlen import attention_paged_ref, attention_varlen_ref

__all__ = ["attention_ref", "attention_bruteforce", "attention_bwd_ref", "kv_head_of",
           "attention_varlen_ref", "attention_paged_ref"]
