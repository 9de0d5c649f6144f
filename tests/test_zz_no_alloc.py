"""The no-allocation split-KV entry point (C: ra_paged_attn_split_noalloc)
against the workspace entry point it shares its kernels with
(ra_paged_attn_split), through the C ABI: bit-identical outputs at the same
split count, on two calls in a row (the second on a smaller input, so its
partial states overwrite only part of what the first left in the scratch
array), and against the oracle. Also: an explicit split count whose partial
states exceed the scratch array is refused before any launch."""

import numpy as np
import pytest
import torch

from tests.parity import DeviceInputs, compare, run_oracle, say
from workloads import make_custom_paged

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_ragged_gqa_amd as ra
    ra.library()


def _noalloc(di, splits):
    import attention_ragged_gqa_amd as ra
    w = di.w
    return ra.ra_paged_attn_split_noalloc(
        di.q, di.q_indptr, di.pages, di.page_indptr, di.page_values, di.length_info,
        sliding_window=w.sliding_window, k_rope_pos_offset=di.k_rope_pos_offset,
        q_rope_position=di.q_rope_position, tree_order_indptr=di.tree_order_indptr,
        tree_order=di.tree_order, causal=w.causal, out=di.out, lse=di.lse, rotary_mode=w.rotary_mode,
        rope_scale=w.rope_scale, rope_theta=w.rope_theta, sm_scale=w.sm_scale, num_kv_splits=splits)


@pytest.mark.parametrize("splits", [5, 0])
def test_noalloc_matches_workspace_entry_point(splits):
    big = make_custom_paged(80, [1, 4, 16, 1, 2, 1], [6000, 3000, 9000, 800, 4000, 2500], h_q=32,
                            h_kv=8, d=128, dtype="bf16", causal=1, store_rope="linear")
    small = make_custom_paged(81, [3, 1], [1500, 700], h_q=16, h_kv=4, d=64, dtype="f16", causal=1)
    for w in (big, small):
        say("[gpu] no-alloc split-KV %s splits=%d" % (w.name, splits))
        di = DeviceInputs(w)
        di.poison()
        out_ws, lse_ws = di.launch(num_kv_splits=splits)
        out_ws, lse_ws = out_ws.clone(), lse_ws.clone()
        di.poison()
        out_na, lse_na = _noalloc(di, splits)
        torch.cuda.synchronize()
        assert torch.equal(out_na, out_ws) and torch.equal(lse_na, lse_ws), "differs from the workspace call"
        ref_out, ref_lse = run_oracle(w)
        d_out, d_lse = compare(out_na, lse_na, ref_out, ref_lse, label="noalloc %s" % w.name)
        say("[gpu] no-alloc %s: max|d out| %.2e max rel|d lse| %.2e" % (w.name, d_out, d_lse))


def test_noalloc_refuses_splits_beyond_the_scratch_array():
    import attention_ragged_gqa_amd as ra
    # 64 splits of 8192 rows x 129 floats = 270 MB of partial states > 32 MiB
    w = make_custom_paged(82, [256, 0], [5000, 64], h_q=32, h_kv=8, d=128, dtype="bf16", causal=1)
    assert ra.ra_paged_attn_split_workspace(w.total_q, w.h_q, w.d, 64) > ra.NOALLOC_SCRATCH_BYTES
    di = DeviceInputs(w)
    with pytest.raises(ra.RagAttnError) as e:
        _noalloc(di, 64)
    assert e.value.status == ra.RA_EINVAL and "scratch" in str(e.value)
    # the automatic count fits itself to the array
    di.poison()
    out, lse = _noalloc(di, 0)
    torch.cuda.synchronize()
    ref_out, ref_lse = run_oracle(w)
    compare(out, lse, ref_out, ref_lse, label="noalloc auto")
