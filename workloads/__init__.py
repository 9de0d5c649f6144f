"""Seeded synthetic inputs for ragged, batched, masked GQA attention.

This package is shared by the test suite, the benchmark and the CPU oracle's
callers. It builds *inputs only*: sequence lengths, random trees with their DFS
enter/exit intervals, page tables (per-head K/V pages or latent pages), length_info arrays and normally distributed
q/k/v values rounded to the storage dtype. It contains none of the attention
arithmetic (no scores, masks, softmax or rotary embedding); both the HIP path
and the oracle compute those on their own.
"""

from .generators import (  # noqa: F401
    CONFIG_NAMES,
    EXTRA_NAMES,
    Workload,
    dfs_intervals,
    make_config,
    make_custom_paged,
    make_custom_ragged,
    make_custom_mla,
    make_custom_tree,
    make_extra,
    mla_pages_from_logical,
    pages_from_logical,
    random_tree,
)
