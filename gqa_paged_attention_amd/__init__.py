"""Grouped-query attention over a paged (HND) KV cache with per-head sinks."""
