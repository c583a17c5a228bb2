"""CPU oracle (test infrastructure): fp64 attention forward (bf16/fp32 and
FP8 forms) and backward.

Only the tests, the package smoke check and the bench's CPU-baseline leg
may import this package.  The product path never does.
"""
from .attention_bwd_fp64 import (attention_bwd_ref, attention_bwd_sampled, backward_flops,
                                 delta_ref)
from .attention_fp8 import attention_fp8_blocked, e4m3_round, fp8_error_bound, fp8_flops
from .attention_fp64 import (algorithmic_flops, attention_ref, default_workers,
                             merge_partials)

__all__ = ["attention_ref", "merge_partials", "default_workers", "algorithmic_flops",
           "attention_bwd_ref", "attention_bwd_sampled", "delta_ref", "backward_flops",
           "attention_fp8_blocked", "e4m3_round", "fp8_error_bound", "fp8_flops"]
