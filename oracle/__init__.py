"""Float64 CPU oracle (test infrastructure only; see oracle/attention.py)."""

from .attention import (  # noqa: F401
    LOG2E,
    MAX_SPLITS,
    SPLIT_ALIGN,
    attention_fwd,
    attention_rows,
    combine,
    decode,
    decode_partials,
    effective_scale,
    kv_head_of,
    max_logit,
    max_logit_rows,
    naive_sink_row_sum_f32,
    query_position,
    rebase_sink_f32,
    split_ranges,
    visible_range,
)
