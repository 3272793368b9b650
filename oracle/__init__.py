"""CPU oracle for Sketch Attention compression -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  It shares no code with the HIP library or its binding.
"""
from .sa_oracle import affinity, assignment, sketch_user, sketch_batch, fold_reference  # noqa: F401
from .refine_oracle import LayerParams, layer_norm, silu, swiglu_ffn, refine_layer, stack_user, stack_batch  # noqa: F401
from .grad_oracle import sketch_grad_user, sketch_grad_batch  # noqa: F401
from .action_oracle import action_fuse  # noqa: F401
