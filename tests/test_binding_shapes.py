"""CPU tests of the Python binding's shape checks: a tensor whose shape does
not match the others is rejected with ValueError before anything reaches the
C ABI or a kernel (the kernels read index arrays and K/V rows at offsets
derived from the sizes they are given, so a mismatch there could read past an
allocation). Host tensors are used on purpose: the shape checks come before
the device checks, so a well-shaped call fails on the device check instead,
which the tests use to show that every case passes the shape checks when
only the named tensor is wrong."""

import pytest
import torch

import attention_ragged_gqa_amd as ra

I32 = torch.int32
F16 = torch.float16


def _tree_args(**over):
    a = dict(q=torch.zeros(10, 8, 128, dtype=F16), q_indptr=torch.tensor([0, 4, 10], dtype=I32),
             k=torch.zeros(10, 2, 128, dtype=F16), v=torch.zeros(10, 2, 128, dtype=F16),
             kv_indptr=torch.tensor([0, 4, 10], dtype=I32), q_rope_position=torch.zeros(10, dtype=I32),
             mn_indptr=torch.tensor([0, 4, 10], dtype=I32), tree_mask=torch.zeros(10, 2, dtype=I32))
    a.update(over)
    return a


def _paged_args(sliding=0, **over):
    b = 2
    a = dict(q=torch.zeros(10, 8, 128, dtype=F16), q_indptr=torch.tensor([0, 4, 10], dtype=I32),
             pages=torch.zeros(6, 2, 2, 16, 128, dtype=F16), page_indptr=torch.tensor([0, 3, 6], dtype=I32),
             page_values=torch.arange(6, dtype=I32),
             length_info=(torch.zeros(3, b, dtype=I32) if sliding else torch.full((b,), 16, dtype=I32)),
             sliding_window=sliding)
    a.update(over)
    return a


def _ragged_args(**over):
    a = dict(q=torch.zeros(10, 8, 64, dtype=F16), q_indptr=torch.tensor([0, 4, 10], dtype=I32),
             k=torch.zeros(12, 4, 64, dtype=F16), v=torch.zeros(12, 4, 64, dtype=F16),
             kv_indptr=torch.tensor([0, 5, 12], dtype=I32))
    a.update(over)
    return a


def _append_args(**over):
    a = dict(k=torch.zeros(7, 2, 128, dtype=F16), v=torch.zeros(7, 2, 128, dtype=F16),
             append_indptr=torch.tensor([0, 3, 7], dtype=I32), append_start=torch.zeros(2, dtype=I32),
             rope_position=torch.zeros(7, dtype=I32), page_indptr=torch.tensor([0, 1, 2], dtype=I32),
             page_values=torch.arange(2, dtype=I32), pages=torch.zeros(2, 2, 2, 16, 128, dtype=F16))
    a.update(over)
    return a


def _shape_error(fn, kwargs):
    with pytest.raises(ValueError) as e:
        fn(**kwargs)
    assert "device tensor" not in str(e.value), "the shape check did not fire: %s" % e.value
    return str(e.value)


def _passes_shape_checks(fn, kwargs):
    with pytest.raises(ValueError, match="device tensor"):
        fn(**kwargs)


def test_well_shaped_calls_reach_the_device_check():
    _passes_shape_checks(ra.ra_tree_attn, dict(_tree_args(), rotary_mode=1))
    _passes_shape_checks(ra.ra_paged_attn, _paged_args())
    _passes_shape_checks(ra.ra_paged_attn, _paged_args(sliding=1))
    _passes_shape_checks(ra.ra_paged_attn_split, _paged_args())
    _passes_shape_checks(ra.ra_ragged_prefill, _ragged_args())
    _passes_shape_checks(ra.ra_paged_kv_append, _append_args())


@pytest.mark.parametrize("over", [
    dict(k=torch.zeros(10, 2, 64, dtype=F16)),                        # head_dim differs from q
    dict(v=torch.zeros(10, 2, 64, dtype=F16)),                        # k and v differ
    dict(k=torch.zeros(10, 3, 128, dtype=F16), v=torch.zeros(10, 3, 128, dtype=F16)),   # 8 % 3
    dict(kv_indptr=torch.tensor([0, 10], dtype=I32)),                 # batch + 1 mismatch
    dict(mn_indptr=torch.tensor([0, 4, 8, 10], dtype=I32)),
    dict(tree_mask=torch.zeros(20, dtype=I32)),                       # not [n, 2]
    dict(q_rope_position=torch.zeros(9, dtype=I32)),                  # not [total_q]
    dict(q=torch.zeros(10, 1024, dtype=F16)),                         # q not 3-d
])
def test_tree_attn_rejects_shapes(over):
    _shape_error(ra.ra_tree_attn, _tree_args(**over))


def test_tree_attn_rope_needs_positions():
    _shape_error(ra.ra_tree_attn, dict(_tree_args(q_rope_position=None), rotary_mode=1))


@pytest.mark.parametrize("fn", [ra.ra_paged_attn, ra.ra_paged_attn_split])
@pytest.mark.parametrize("sliding,over", [
    (0, dict(pages=torch.zeros(6, 2, 2, 16, 64, dtype=F16))),         # head_dim differs
    (0, dict(pages=torch.zeros(6, 3, 2, 16, 128, dtype=F16))),        # not K|V pairs
    (0, dict(pages=torch.zeros(6, 2, 3, 16, 128, dtype=F16))),        # 8 % 3
    (0, dict(page_indptr=torch.tensor([0, 6], dtype=I32))),
    (0, dict(length_info=torch.zeros(3, dtype=I32))),                 # [b] expected
    (1, dict(length_info=torch.zeros(2, dtype=I32))),                 # [3, b] expected
    (1, dict(length_info=torch.zeros(3, 3, dtype=I32))),
    (0, dict(k_rope_pos_offset=torch.zeros(3, dtype=I32))),
    (0, dict(q_rope_position=torch.zeros(11, dtype=I32))),
    (0, dict(tree_order=torch.zeros(10, 2, dtype=I32))),              # without its indptr
    (0, dict(tree_order_indptr=torch.tensor([0, 4, 10], dtype=I32), tree_order=torch.zeros(10, dtype=I32))),
    (0, dict(tree_order_indptr=torch.tensor([0, 10], dtype=I32), tree_order=torch.zeros(10, 2, dtype=I32))),
])
def test_paged_attn_rejects_shapes(fn, sliding, over):
    _shape_error(fn, _paged_args(sliding=sliding, **over))


def test_paged_attn_rope_needs_positions():
    _shape_error(ra.ra_paged_attn, dict(_paged_args(), rotary_mode=1))


@pytest.mark.parametrize("over", [
    dict(k=torch.zeros(12, 4, 128, dtype=F16), v=torch.zeros(12, 4, 128, dtype=F16)),
    dict(v=torch.zeros(11, 4, 64, dtype=F16)),
    dict(kv_indptr=torch.tensor([0, 5, 9, 12], dtype=I32)),
    dict(valid_len=torch.zeros(3, dtype=I32), pad_mode=1, causal=0),
    dict(pad_mode=2),                                                  # valid_len missing
])
def test_ragged_prefill_rejects_shapes(over):
    _shape_error(ra.ra_ragged_prefill, _ragged_args(**over))


@pytest.mark.parametrize("over", [
    dict(k=torch.zeros(7, 2, 64, dtype=F16), v=torch.zeros(7, 2, 64, dtype=F16)),
    dict(k=torch.zeros(7, 4, 128, dtype=F16), v=torch.zeros(7, 4, 128, dtype=F16)),
    dict(v=torch.zeros(6, 2, 128, dtype=F16)),
    dict(append_start=torch.zeros(3, dtype=I32)),
    dict(page_indptr=torch.tensor([0, 2], dtype=I32)),
    dict(rope_position=torch.zeros(8, dtype=I32)),
    dict(pages=torch.zeros(2, 2, 16, 128, dtype=F16)),
])
def test_append_rejects_shapes(over):
    _shape_error(ra.ra_paged_kv_append, _append_args(**over))


def _mla_args(**over):
    a = dict(q=torch.zeros(10, 16, 576, dtype=F16), q_indptr=torch.tensor([0, 4, 10], dtype=I32),
             pages=torch.zeros(5, 16, 576, dtype=F16), page_indptr=torch.tensor([0, 2, 5], dtype=I32),
             page_values=torch.arange(5, dtype=I32), last_page_len=torch.tensor([3, 16], dtype=I32))
    a.update(over)
    return a


def test_mla_well_shaped_call_reaches_the_device_check():
    _passes_shape_checks(ra.ra_mla_paged_prefill, _mla_args())


@pytest.mark.parametrize("over", [
    dict(pages=torch.zeros(5, 16, 512, dtype=F16)),                   # d_qk differs from q
    dict(pages=torch.zeros(5, 2, 16, 576, dtype=F16)),                # per-head K/V pages
    dict(page_indptr=torch.tensor([0, 5], dtype=I32)),
    dict(last_page_len=torch.tensor([3], dtype=I32)),
    dict(last_page_len=None),
    dict(d_latent=600),
    dict(q=torch.zeros(10, 576, dtype=F16)),
])
def test_mla_rejects_shapes(over):
    _shape_error(ra.ra_mla_paged_prefill, _mla_args(**over))
