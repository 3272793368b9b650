"""MI355X-native Sketch Attention compression (SequenceO1 cache-miss path).

The computation lives in libsa.so (hand-written HIP for gfx950, C ABI in
include/sa.h); this package holds its thin binding and the seeded synthetic
workloads.  The library itself is loaded on first use, so the workloads can
be used without it; any call into the binding fails loudly when it is absent.
"""
from .binding import (  # noqa: F401
    ActionFusion,
    SAError,
    SketchAttention,
    SketchAttentionGrad,
    SketchStack,
    sa_action_check_config,
    sa_action_compress_batch,
    sa_action_create,
    sa_action_destroy,
    sa_action_fuse,
    sa_check_batch,
    sa_check_config,
    sa_compress_batch,
    sa_compress_batch_bound,
    sa_compress_batch_noalloc,
    sa_create,
    sa_describe_plan,
    sa_destroy,
    sa_get_folded,
    sa_grad_check_config,
    sa_grad_compute,
    sa_grad_create,
    sa_grad_destroy,
    sa_measure_ceilings,
    sa_read_kernel_timing,
    sa_reserve,
    sa_set_kernel_timing,
    sa_stack_compress_batch,
    sa_stack_compress_batch_bound,
    sa_stack_create,
    sa_stack_destroy,
    sa_status_string,
)
