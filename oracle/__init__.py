"""Float64 CPU oracle for shared-QK LSH self-attention and local attention
(test infrastructure only).

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package; the library itself never does.
"""
from .lsh_oracle import (  # noqa: F401
    attend_positions,
    chunk_attention_round,
    combine_rounds,
    exact_projection_margin,
    lsh_attention,
    lsh_attention_head,
    lsh_hash,
    lsh_sort,
)
from .local_oracle import (  # noqa: F401
    local_attention,
    local_attention_head,
    local_window,
)
from .backward_oracle import (  # noqa: F401
    dense_forward,
    grad_positions,
    lsh_attention_head_grad,
    target_counts,
)
from .ff_oracle import (  # noqa: F401
    chunked_feed_forward,
    feed_forward,
)
