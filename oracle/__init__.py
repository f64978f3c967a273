"""CPU fp64 oracle for causal multi-head / grouped-query attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it, to check and to time the
GPU kernels.  It imports NumPy and nothing else, and shares no code, table or
constant with the HIP library.

What it computes is attention written out by its definition, with the score
matrix materialised and a plain (non-blockwise) softmax over each row: the
"naive" attention backend of the RoseLLM README ("Systems highlights",
"Inference and serving") and the ScaledDotProductAttention / Softmax
primitives of the llm-from-scratch "Project Overview" page ("Core Stack:
llm/", transformer.py).  The blockwise online softmax that the GPU kernels use
("Performance Layer: kernel/ and parallel/") reaches the same values without
materialising the scores, so this definition is the thing to match.

Every public function is pinned by ``tests/test_oracle.py`` against closed
forms, invariants, an independent library routine and a 50-digit brute force
(see that file); ``tests/test_oracle_mutants.py`` plants mistakes in this
source and checks that the pins catch each one.
"""

from .attention import (  # noqa: F401
    decode_paged,
    decode_paged_append,
    decode_paged_fp8,
    fp8_e4m3_value,
    gather_pages,
    kv_append,
    kv_head_of,
    prefill,
    prefill_paged,
    prefill_paged_append,
    prefill_varlen,
    prefill_rows,
)
