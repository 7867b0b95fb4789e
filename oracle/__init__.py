"""CPU oracle for the sparse-weight matmul path -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check of the package entry file and the bench's
cpu_baseline leg may import anything here.  The GPU library never calls it and
it never calls the GPU library: the two share no code, headers, tables or
helpers.  The only common module is the seeded input generator
(``swm_workloads``), which holds none of the method's arithmetic.

Contents
--------
``reference``  plain fp64 definition of the product of a pruned weight matrix
               and dense activations, with and without zero-activation skipping.
``tcb``        an independent numpy encoder / decoder of the tiled
               column-bitmap format (SWM-TCB v1), written from its spec.
``exact``      exact integer brute force used to pin the fp64 reference.
``colruns``    an independent numpy encoder / decoder of the column-run
               encoding (SWM-CR v2) used by activation skipping.

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` against closed forms, brute force, hand-worked
format bytes and invariants.  The pages print no worked numeric example, so no
pin compares against a value printed on the pages themselves.
"""
from .reference import (masked_matmul, masked_matmul_skip, active_inputs, to_fp16, threshold_activations,
                        masked_matmul_threshold, silu, gate_up_silu)
from .tcb import tcb_encode, tcb_decode, tcb_parse, TcbFormat
from .exact import exact_masked_matmul, fp64_error_bound
from .colruns import colruns_encode, colruns_parse, colruns_decode, ColRuns

__all__ = [
    "masked_matmul", "masked_matmul_skip", "active_inputs", "to_fp16", "threshold_activations", "masked_matmul_threshold",
    "silu", "gate_up_silu",
    "tcb_encode", "tcb_decode", "tcb_parse", "TcbFormat",
    "exact_masked_matmul", "fp64_error_bound",
    "colruns_encode", "colruns_parse", "colruns_decode", "ColRuns",
]
