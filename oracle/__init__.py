"""CPU fp64 oracle for exact masked attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the HIP path.
"""
from .masked_attention import (attention, probabilities, blockwise_attention_rows, visible,
                        mask_rows, visible_pairs_bruteforce, useful_flops)
from .masked_attention_bwd import attention_backward, delta_rows
from .decode import decode, cache_to_sequence, slot_of

__all__ = ["attention", "probabilities", "blockwise_attention_rows", "visible",
           "mask_rows", "visible_pairs_bruteforce", "useful_flops",
           "attention_backward", "delta_rows", "decode", "cache_to_sequence", "slot_of"]
