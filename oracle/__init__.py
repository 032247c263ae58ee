"""fp64 CPU oracle for the ARL2 hybrid attention step.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It shares no code
with the HIP path and imports nothing from it.
"""
from .arl2_oracle import (  # noqa: F401
    L2_EPS,
    attention_logsumexp,
    attention_weights,
    commit,
    commit_backward,
    commit_inputs,
    default_scale,
    feature_map,
    fullkv_attention,
    hybrid_stack_rollout,
    inter_read,
    intra_attention,
    intra_attention_backward,
    l2_normalize_rows,
    read,
    read_backward,
    rollout,
    rollout_backward,
    softmax_layer_rollout,
    state_commit,
    state_scan,
    token_level_read,
    token_level_rollout,
)
