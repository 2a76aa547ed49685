"""fp64 CPU oracle for the memory-bounded MoE layer (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls it, and shares no code with it.
"""

from .moe_oracle import (  # noqa: F401
    plan_chunks,
    chunk_sizes,
    chunk_tokens,
    pair_base,
    router_logits,
    topk_select,
    gates_from_logits,
    route,
    permute_chunk,
    silu,
    expert_ffn,
    moe_forward,
    forward_tokens,
    moe_backward,
    expert_grads,
    router_grads,
    backward_tokens,
    logit_error_bound,
    dispatch_bound_bytes,
)

from .ce_oracle import (  # noqa: F401,E402
    ce_strips,
    strip_bound_bytes,
    ce_logits,
    ce_forward,
    ce_fold_strips,
    ce_dlogits,
    ce_backward,
    ce_forward_tokens,
    ce_backward_tokens,
    ce_backward_tokens_rows,
)
