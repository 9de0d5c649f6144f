"""Plant plausible mistakes in the CPU oracle and check the pins catch each one.

Each mutation monkeypatches one oracle function with a wrong variant; at
least one pin in ``test_oracle_pins`` must then fail. Mistakes are planted in
the oracle only, on the CPU.
"""

import numpy as np
import pytest

import oracle
import oracle.attention as OA
from tests import test_oracle_pins as P

PINS = [
    P.test_golden_two_key_closed_form,
    P.test_golden_tree6_intervals,
    P.test_ones_v_gives_ones,
    P.test_singleton_forest_gives_v_and_score,
    P.test_lse_is_base2_logsumexp,
    P.test_causal_matches_sdpa_bottom_right,
    P.test_noncausal_matches_sdpa_full,
    P.test_tree_matches_sdpa_with_ancestor_sets,
    lambda: P.test_exhaustive_small_trees(4),
    P.test_chain_tree_equals_causal,
    P.test_all_prefix_tree_equals_full_attention,
    P.test_paged_tree_prefix_plus_ancestors,
    P.test_gqa_equals_replicated_kv,
    P.test_rope_is_complex_rotation_of_halves,
    P.test_rope_frequencies_closed_form,
    P.test_rope_norm_and_identity,
    lambda: P.test_rope_rounded_within_half_ulp("bf16"),
    P.test_sliding_window_equals_causal_on_sink_plus_window,
    P.test_cache_rope_equals_prerotated_pages,
    P.test_empty_rows_and_sequences,
    P.test_rope_relative_position_invariance,
    P.test_inkernel_k_rope_equals_cache_rope_at_offset,
    lambda: P.test_mla_matches_sdpa_on_expanded_heads(1),
    P.test_mla_absorbed_equals_mha_with_up_projections,
    P.test_mla_single_visible_key_gives_latent_row,
]

_orig_attend = OA.attend
_orig_tree_visible = OA.tree_visible
_orig_causal_visible = OA.causal_visible
_orig_rope_angles = OA._rope_angles
_orig_seq_offset = OA.seq_offset
_orig_kv_chunk_len = OA.kv_chunk_len


def _attend_no_scale(qr, kr, vr, vis, sm_scale):
    return _orig_attend(qr, kr, vr, vis, 1.0)


def _attend_natural_log(qr, kr, vr, vis, sm_scale):
    o, l = _orig_attend(qr, kr, vr, vis, sm_scale)
    return o, l * OA.LN2


def _attend_k_as_v(qr, kr, vr, vis, sm_scale):
    return _orig_attend(qr, kr, kr, vis, sm_scale)


def _attend_sequence_mod_heads(qb, tok_global, qi, kseq, vseq, vis, h_q, h_kv, sm_scale, out, lse):
    for h in range(h_q):
        o, l = _orig_attend(qb[:, h, :], kseq[:, h % h_kv, :], vseq[:, h % h_kv, :], vis, sm_scale)
        out[tok_global, h, :] = o
        lse[tok_global, h] = l


def _tree_descendants(order, rows, kv_len, qo_len):
    order = np.asarray(order).reshape(-1, 2)
    swapped = order.copy()
    vis = _orig_tree_visible(order, rows, kv_len, qo_len)
    tree_len = order.shape[0]
    ts = kv_len - tree_len
    c = np.clip(np.asarray(rows) + tree_len - qo_len, 0, max(tree_len - 1, 0))
    if tree_len:
        p = np.arange(tree_len)
        # descendant test: enter[p] in [enter[c], exit[c])
        vis[:, ts:] = (swapped[p, 0][None, :] >= swapped[c, 0][:, None]) & (swapped[p, 0][None, :] < swapped[c, 1][:, None])
    return vis


def _causal_top_left(rows, kv_len, qo_len, causal=1):
    cols = np.arange(kv_len)[None, :]
    r = np.asarray(rows)[:, None]
    return (cols < r + 1) if causal > 0 else _orig_causal_visible(rows, kv_len, qo_len, causal)


def _rope_angles_wrong_freq(pos, d, theta, scale):
    k = np.arange(d // 2, dtype=np.float64)
    return (np.asarray(pos, np.float64) * scale)[:, None] * np.power(theta, -1.0 * k / d)[None, :]


def _rope_exact_interleaved(x, pos, theta, scale):
    x = OA._f64(x)
    d = x.shape[-1]
    ang = _orig_rope_angles(pos, d, theta, scale)[:, None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x1 * c - x2 * s
    y[..., 1::2] = x2 * c + x1 * s
    return y


def _rope_exact_wrong_sign(x, pos, theta, scale):
    x = OA._f64(x)
    d = x.shape[-1]
    h = d // 2
    ang = _orig_rope_angles(pos, d, theta, scale)[:, None, :]
    c, s = np.cos(ang), np.sin(ang)
    return np.concatenate([x[..., :h] * c + x[..., h:] * s, x[..., h:] * c - x[..., :h] * s], axis=-1)


def _rope_rounded_wrong_sign(x, pos, theta, scale, dtype):
    y = _rope_exact_wrong_sign(x, pos, theta, scale).astype(np.float32)
    return OA._round_f32_to(y, dtype)


def _rope_rounded_interleaved(x, pos, theta, scale, dtype):
    return OA._round_f32_to(_rope_exact_interleaved(x, pos, theta, scale).astype(np.float32), dtype)


def _rope_rounded_identity(x, pos, theta, scale, dtype):
    return OA._f64(x)


def _seq_offset_plus_sink(j, b, length_info, sliding_window):
    j = np.asarray(j)
    if not sliding_window:
        return j
    li = np.asarray(length_info)
    sink, off = int(li[2, b]), int(li[1, b])
    return np.where(j < sink, j, j + off)          # forgot to subtract the sink


def _attend_latent_v_from_last_columns(qr, kr, vr, vis, sm_scale):
    # latent attention (V narrower than K): V taken from the last columns
    if vr.shape[1] < kr.shape[1]:
        vr = kr[:, kr.shape[1] - vr.shape[1]:]
    return _orig_attend(qr, kr, vr, vis, sm_scale)


def _attend_latent_k_without_rope_columns(qr, kr, vr, vis, sm_scale):
    # latent attention: scores over the latent columns only
    if vr.shape[1] < kr.shape[1]:
        n = vr.shape[1]
        return _orig_attend(qr[:, :n], kr[:, :n], vr, vis, sm_scale)
    return _orig_attend(qr, kr, vr, vis, sm_scale)


def _kv_chunk_len_no_sink(b, page_indptr, length_info, sliding_window):
    n = _orig_kv_chunk_len(b, page_indptr, length_info, sliding_window)
    if sliding_window and n:
        n -= int(np.asarray(length_info)[2, b])
    return n


MUTATIONS = {
    "drop_sm_scale": [("attend", _attend_no_scale)],
    "natural_log_lse": [("attend", _attend_natural_log)],
    "k_used_as_v": [("attend", _attend_k_as_v)],
    "kv_head_h_mod_hkv": [("_attend_sequence", _attend_sequence_mod_heads)],
    "tree_descendants": [("tree_visible", _tree_descendants)],
    "causal_top_left": [("causal_visible", _causal_top_left)],
    "rope_wrong_frequency": [("_rope_angles", _rope_angles_wrong_freq)],
    "rope_interleaved_pairs": [("rope_exact", _rope_exact_interleaved)],
    "rope_wrong_sign": [("rope_exact", _rope_exact_wrong_sign), ("rope", _rope_rounded_wrong_sign)],
    "rope_rounded_interleaved": [("rope", _rope_rounded_interleaved)],
    "rope_skipped": [("rope", _rope_rounded_identity)],
    "sliding_offset": [("seq_offset", _seq_offset_plus_sink)],
    "chunk_len_no_sink": [("kv_chunk_len", _kv_chunk_len_no_sink)],
    "latent_v_from_last_columns": [("attend", _attend_latent_v_from_last_columns)],
    "latent_scores_without_rope_columns": [("attend", _attend_latent_k_without_rope_columns)],
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    for attr, fn in MUTATIONS[name]:
        monkeypatch.setattr(OA, attr, fn)
        if hasattr(oracle, attr):
            monkeypatch.setattr(oracle, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            failed.append(getattr(pin, "__name__", "lambda"))
    assert failed, "mutation %s survived every pin" % name
