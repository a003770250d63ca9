"""fp64 CPU oracle of the DFlash2 draft-block path (test infrastructure only).

Only the tests, the smoke check and the bench's CPU-baseline leg use this
package; the product path never imports it.  It loads ``liboracle.so`` (plain
C, see ``oracle.c``) and exposes numpy-level wrappers.  Inputs are the raw
tensors the generators produce: fp32 arrays, or bf16 bit patterns as uint16.
"""
from .api import (  # noqa: F401
    load,
    conv,
    round_to,
    head,
    topk,
    transitions,
    viterbi,
    walk,
    draft_block,
    threads,
)
