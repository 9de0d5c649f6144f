"""CPU oracle for ragged, batched, masked GQA attention.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The HIP library never calls it, and it shares no code with the HIP
path: it imports neither ``attention_ragged_gqa_amd`` nor its C library.

The oracle is the plain definition of what the attention operators on the TVM
pages compute (page "relax/frontend/nn/llm/_kernel_common.py": ``_rope``,
``_causal_mask``, ``_get_kv_chunk_len``, ``_get_seq_offset`` and the prefill
macros; page "relax/frontend/nn/llm/tree_attn.py": ``_check_tree_order`` and the
CPU tree-attention kernel), written in float64 numpy without tiling: scores,
masked softmax, weighted V sum and base-2 log-sum-exp. Where the pages fix a
precision it follows them: the rotary embedding is evaluated in float32 and
rounded to the storage dtype.

Modules:
  attention -- vectorised float64 oracle (tree_attn, paged_attn,
               ragged_prefill with padded masks, mla_paged_attn over a
               latent cache, rope, masks, merge_states for split key sets)
  scalar    -- pure-Python brute force for tiny inputs (ancestor sets from
               parent pointers rather than DFS intervals)
"""

from .attention import (  # noqa: F401
    LN2,
    attend,
    causal_visible,
    kv_chunk_len,
    merge_states,
    mla_paged_attn,
    padded_visible,
    paged_attn,
    ragged_prefill,
    rope,
    rope_exact,
    seq_offset,
    tree_attn,
    tree_visible,
)
