"""fp64 CPU oracle for exact attention — test infrastructure only.

Only the tests, the smoke check and the bench's CPU-baseline leg use this package; the
product path (the HIP library and its binding) never imports or calls it.
"""
from .attention import (  # noqa: F401
    forward, forward_kv, forward_blocksparse, forward_varlen, forward_rows, backward, backward_kv,
    backward_blocksparse, backward_varlen, decode, decode_multi, probabilities, split_kv_decode, lse_merge, attention_flops, upcast,
)
