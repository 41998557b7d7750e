"""CPU oracle for paged attention (test infrastructure only; see
paged_attention.py).  Only tests, the smoke check and the benchmark's CPU
baseline may import it."""
from .paged_attention import (gather, attend, paged_attention, query_positions, q_row_starts,
                              split_page_ranges, pages_per_split_even, split_partials, merge)
from .kv_append import append_kv, copy_pages

__all__ = ["gather", "attend", "paged_attention", "query_positions", "q_row_starts",
           "split_page_ranges", "pages_per_split_even", "split_partials", "merge", "append_kv",
           "copy_pages"]
