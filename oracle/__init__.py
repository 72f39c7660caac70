"""Float64 CPU oracle for exact softmax attention (test infrastructure only:
imported by the tests, the smoke check and the benchmark's CPU-baseline leg,
never by the product path)."""
from .attention_oracle import (  # noqa: F401
    attention_state,
    backward_dkdv_cols,
    backward_dq_rows,
    causal_blocked,
    chunkwise_unrescaled,
    dense_backward,
    decode_forward,
    dense_forward,
    forward_rows,
    merge_states,
    online_softmax_step,
    tiled_forward,
)
