"""fp64 CPU oracle for sink attention -- TEST INFRASTRUCTURE.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package. It shares no code with softmax_sink_amd (the HIP path)
and imports nothing from it.
"""
from .sink_attention import (  # noqa: F401
    keep_mask, keep_row, keep_mask_top_left, sink_attention_forward,
    sink_attention_backward, sink_attention_dsink, sink_attention_rows, sink_logit_for_n,
    softmax_n, classify_tiles, forward_items, backward_items, decode_items,
    count_kept_pairs, gather_paged, merge_partials, DEAD, PARTIAL, FULL,
)
