"""Pins for the CPU oracle: each checks it against something other than itself.

Every test here is CPU-only. The pins are chosen so that a plausible mistake
in the oracle (a dropped sm_scale, a natural-log lse, a transposed operand, a
wrong KV-head mapping, a descendant-instead-of-ancestor tree test, a
top-left causal mask, a wrong RoPE pairing, sign or frequency, a wrong page
or sliding-window index) fails at least one of them; ``test_oracle_mutations``
plants such mistakes and checks that.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import scalar
from workloads import dfs_intervals, make_config, make_custom_paged, make_custom_tree, pages_from_logical

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _sdpa(q, k, v, mask, scale):
    """torch CPU scaled_dot_product_attention in float64.
    q [R, H, D], k/v [L, H, D], mask [R, L] bool (True = visible)."""
    qt = torch.as_tensor(q, dtype=torch.float64).permute(1, 0, 2)[None]
    kt = torch.as_tensor(k, dtype=torch.float64).permute(1, 0, 2)[None]
    vt = torch.as_tensor(v, dtype=torch.float64).permute(1, 0, 2)[None]
    m = torch.as_tensor(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def _expand_kv(x, g):
    return np.repeat(np.asarray(x, dtype=np.float64), g, axis=1)


def _ancestor_mask(parent):
    n = len(parent)
    m = np.zeros((n, n), dtype=bool)
    for c in range(n):
        for p in scalar.ancestors_or_self(parent, c):
            m[c, p] = True
    return m


def _tree_oracle(w, **kw):
    return oracle.tree_attn(w.q, w.q_indptr, w.k, w.v, w.kv_indptr, w.q_rope_position, w.mn_indptr,
                            w.tree_mask, w.rotary_mode, w.rope_scale, w.rope_theta, w.sm_scale,
                            w.dtype, **kw)


def _paged_oracle(w, pages=None, **kw):
    pages = pages_from_logical(w) if pages is None else pages
    args = dict(tree_order_indptr=w.tree_order_indptr, tree_order=w.tree_order,
                q_rope_position=w.q_rope_position, k_rope_pos_offset=w.k_rope_pos_offset,
                rotary_mode=w.rotary_mode, rope_scale=w.rope_scale, rope_theta=w.rope_theta)
    if w.store_rope_position is not None:
        args.update(cache_rope_position=w.store_rope_position, cache_rope_indptr=w.kv_store_indptr)
    args.update(kw)
    return oracle.paged_attn(w.q, w.q_indptr, pages, w.page_indptr, w.page_values, w.length_info,
                             w.sliding_window, w.causal, w.sm_scale, w.dtype, **args)


# ---------------------------------------------------------------------------
# golden, hand-worked examples
# ---------------------------------------------------------------------------

def test_golden_two_key_closed_form():
    g = json.load(open(os.path.join(GOLDEN, "two_key_closed_form.json")))
    q = np.array(g["q"], float)[:, None, :]
    k = np.array(g["k"], float)[:, None, :]
    v = np.array(g["v"], float)[:, None, :]
    ip = np.array([0, 2], np.int32)
    out, lse = oracle.tree_attn(q, ip, k, v, ip, None, ip, np.array(g["enter_exit"]), 0, 1.0, 1e4, 1.0, "f16")
    np.testing.assert_allclose(out[:, 0, :], g["expected"]["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[:, 0], g["expected"]["lse"], rtol=0, atol=1e-12)


def test_golden_tree6_intervals():
    g = json.load(open(os.path.join(GOLDEN, "tree6_intervals.json")))
    iv = dfs_intervals(np.array(g["parent"], np.int32))
    assert iv[:, 0].tolist() == g["enter"]
    assert iv[:, 1].tolist() == g["exit"]
    vis = oracle.tree_visible(iv, np.arange(6), 6, 6)
    for c, keys in enumerate(g["visible_keys_of_query"]):
        assert np.flatnonzero(vis[c]).tolist() == keys


# ---------------------------------------------------------------------------
# softmax / lse
# ---------------------------------------------------------------------------

def test_ones_v_gives_ones():
    w = make_custom_tree(7, [9, 33, 1], h_q=4, h_kv=2, d=64, dtype="f16")
    w.v = torch.ones_like(w.v)
    out, _ = _tree_oracle(w)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-12)


def test_singleton_forest_gives_v_and_score():
    """Every node its own root: row i sees key i only -> out = v_i, lse = s_ii / ln2."""
    w = make_custom_tree(8, [12, 5], h_q=4, h_kv=2, d=64, dtype="bf16")
    n = w.total_q
    w.tree_mask = np.stack([np.r_[0:12, 0:5], np.r_[1:13, 1:6]], axis=1).astype(np.int32)
    out, lse = _tree_oracle(w)
    q = w.q.double().numpy()
    k = w.k.double().numpy()
    v = w.v.double().numpy()
    for i in range(n):
        for h in range(4):
            s = w.sm_scale * math.fsum(q[i, h] * k[i, h // 2])
            np.testing.assert_allclose(out[i, h], v[i, h // 2], rtol=0, atol=1e-12)
            assert abs(lse[i, h] - s / math.log(2)) < 1e-12


def test_spread_closed_forms():
    """The spread the oracle reports for tolerances, against closed forms:
    zero queries give equal weights over the visible keys, so the spread is
    the population standard deviation of v over them (numpy std); a row that
    sees one key has spread 0; paged and ragged entry points agree with the
    same definition."""
    rng = np.random.default_rng(12)
    L, d = 37, 16
    v = rng.standard_normal((L, d))
    vis = np.ones((3, L), dtype=bool)
    vis[1, 20:] = False                       # row 1 sees keys 0..19
    vis[2, 1:] = False                        # row 2 sees key 0 only
    out, _, sd = oracle.attend(np.zeros((3, d)), rng.standard_normal((L, d)), v, vis, 0.5, spread=True)
    np.testing.assert_allclose(sd[0], v.std(axis=0), rtol=0, atol=1e-12)
    np.testing.assert_allclose(sd[1], v[:20].std(axis=0), rtol=0, atol=1e-12)
    np.testing.assert_allclose(sd[2], 0.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out[1], v[:20].mean(axis=0), rtol=0, atol=1e-12)
    # the entry points fill it where they fill out, from the same weights
    w = make_custom_tree(14, [9, 33, 1], h_q=4, h_kv=2, d=64, dtype="f16")
    w.q = torch.zeros_like(w.q)
    sp = np.full(w.q.shape, np.nan)
    out_t, _ = oracle.tree_attn(w.q, w.q_indptr, w.k, w.v, w.kv_indptr, None, w.mn_indptr, w.tree_mask,
                                0, 1.0, 1e4, w.sm_scale, w.dtype, spread=sp)
    v64 = w.v.double().numpy()
    order = np.asarray(w.tree_mask)
    for r in range(w.total_q):
        b = int(np.searchsorted(np.asarray(w.q_indptr), r, side="right") - 1)
        k0 = int(w.kv_indptr[b])
        mine = order[int(w.mn_indptr[b]):int(w.mn_indptr[b + 1])]
        c = r - int(w.q_indptr[b])
        anc = [k0 + j for j in range(len(mine)) if mine[j, 0] <= mine[c, 0] < mine[j, 1]]
        for h in range(4):
            np.testing.assert_allclose(sp[r, h], v64[anc, h // 2].std(axis=0), rtol=0, atol=1e-9)


def test_lse_is_base2_logsumexp():
    w = make_custom_tree(9, [20, 31], h_q=4, h_kv=2, d=64, dtype="f16", max_children=3)
    out, lse = _tree_oracle(w)
    q = torch.as_tensor(w.q, dtype=torch.float64)
    k = torch.as_tensor(w.k, dtype=torch.float64)
    for b, par in enumerate(w.parents):
        base = int(w.q_indptr[b])
        am = _ancestor_mask(par)
        for c in range(len(par)):
            for h in range(4):
                s = (k[base:base + len(par), h // 2] @ q[base + c, h]).numpy() * w.sm_scale
                ref = scipy.special.logsumexp(s[am[c]]) / math.log(2)
                assert abs(lse[base + c, h] - ref) < 1e-10


# ---------------------------------------------------------------------------
# masks against a textbook routine / brute force
# ---------------------------------------------------------------------------

def test_causal_matches_sdpa_bottom_right():
    qo, pre = [37, 64, 5], [63, 0, 100]
    w = make_custom_paged(10, qo, [a + b for a, b in zip(qo, pre)], h_q=8, h_kv=2, d=64,
                          dtype="bf16", causal=1)
    out, lse = _paged_oracle(w)
    for b in range(3):
        q0, q1 = int(w.q_indptr[b]), int(w.q_indptr[b + 1])
        s0, s1 = int(w.kv_store_indptr[b]), int(w.kv_store_indptr[b + 1])
        L = s1 - s0
        mask = torch.ones(q1 - q0, L, dtype=torch.bool).tril(diagonal=L - (q1 - q0))
        ref = _sdpa(w.q[q0:q1].double(), _expand_kv(w.k_store[s0:s1].double(), 4),
                    _expand_kv(w.v_store[s0:s1].double(), 4), mask.numpy(), w.sm_scale)
        np.testing.assert_allclose(out[q0:q1], ref, rtol=0, atol=1e-10)


def test_noncausal_matches_sdpa_full():
    w = make_custom_paged(11, [17, 3], [40, 3], h_q=4, h_kv=4, d=128, dtype="f16", causal=0)
    out, _ = _paged_oracle(w)
    for b in range(2):
        q0, q1 = int(w.q_indptr[b]), int(w.q_indptr[b + 1])
        s0, s1 = int(w.kv_store_indptr[b]), int(w.kv_store_indptr[b + 1])
        mask = np.ones((q1 - q0, s1 - s0), bool)
        ref = _sdpa(w.q[q0:q1].double(), w.k_store[s0:s1].double(), w.v_store[s0:s1].double(), mask, w.sm_scale)
        np.testing.assert_allclose(out[q0:q1], ref, rtol=0, atol=1e-10)


def test_tree_matches_sdpa_with_ancestor_sets():
    w = make_custom_tree(12, [1, 13, 40], h_q=8, h_kv=2, d=64, dtype="f16", max_children=4)
    out, _ = _tree_oracle(w)
    for b, par in enumerate(w.parents):
        q0, q1 = int(w.q_indptr[b]), int(w.q_indptr[b + 1])
        ref = _sdpa(w.q[q0:q1].double(), _expand_kv(w.k[q0:q1].double(), 4),
                    _expand_kv(w.v[q0:q1].double(), 4), _ancestor_mask(par), w.sm_scale)
        np.testing.assert_allclose(out[q0:q1], ref, rtol=0, atol=1e-10)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_exhaustive_small_trees(n):
    """Every tree on n nodes in generation order: interval test == ancestor sets."""
    for choice in itertools.product(*[range(i) for i in range(1, n)]):
        parent = np.array((-1,) + choice, np.int32)
        vis = oracle.tree_visible(dfs_intervals(parent), np.arange(n), n, n)
        assert (vis == _ancestor_mask(parent)).all(), parent


def test_chain_tree_equals_causal():
    n = 29
    w = make_custom_tree(13, [n], h_q=4, h_kv=1, d=64, dtype="bf16")
    w.tree_mask = dfs_intervals(np.arange(-1, n - 1, dtype=np.int32))
    out, lse = _tree_oracle(w)
    mask = np.tril(np.ones((n, n), bool))
    ref = _sdpa(w.q.double(), _expand_kv(w.k.double(), 4), _expand_kv(w.v.double(), 4), mask, w.sm_scale)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-10)


def test_all_prefix_tree_equals_full_attention():
    """Paged tree whose every interval is [0, n): every column visible."""
    w = make_custom_paged(14, [9], [30], h_q=4, h_kv=2, d=64, dtype="bf16", causal=0, tree=True)
    w.tree_order = np.tile(np.array([[0, 9]], np.int32), (9, 1))
    out, _ = _paged_oracle(w)
    ref = _sdpa(w.q.double(), _expand_kv(w.k_store.double(), 2), _expand_kv(w.v_store.double(), 2),
                np.ones((9, 30), bool), w.sm_scale)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-10)


def test_paged_tree_prefix_plus_ancestors():
    w = make_custom_paged(15, [6, 11], [6 + 20, 11 + 3], h_q=4, h_kv=2, d=64, dtype="f16",
                          causal=0, tree=True, tree_max_children=2)
    out, _ = _paged_oracle(w)
    for b in range(2):
        q0, q1 = int(w.q_indptr[b]), int(w.q_indptr[b + 1])
        s0, s1 = int(w.kv_store_indptr[b]), int(w.kv_store_indptr[b + 1])
        n, L = q1 - q0, s1 - s0
        mask = np.zeros((n, L), bool)
        mask[:, : L - n] = True
        mask[:, L - n:] = _ancestor_mask(w.parents[b])
        ref = _sdpa(w.q[q0:q1].double(), _expand_kv(w.k_store[s0:s1].double(), 2),
                    _expand_kv(w.v_store[s0:s1].double(), 2), mask, w.sm_scale)
        np.testing.assert_allclose(out[q0:q1], ref, rtol=0, atol=1e-10)


# ---------------------------------------------------------------------------
# GQA
# ---------------------------------------------------------------------------

def test_gqa_equals_replicated_kv():
    w = make_custom_tree(16, [10, 23], h_q=8, h_kv=2, d=64, dtype="f16", max_children=4)
    out, lse = _tree_oracle(w)
    w.k = w.k.repeat_interleave(4, dim=1)
    w.v = w.v.repeat_interleave(4, dim=1)
    out2, lse2 = _tree_oracle(w)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


# ---------------------------------------------------------------------------
# rotary embedding
# ---------------------------------------------------------------------------

def test_rope_is_complex_rotation_of_halves():
    rng = np.random.default_rng(0)
    d = 128
    x = rng.standard_normal((7, 3, d))
    pos = np.array([0, 1, 5, 100, 4097, 20000, 123456])
    y = oracle.rope_exact(x, pos, 5e5, 1.0)
    k = np.arange(d // 2)
    inv = 5e5 ** (-2.0 * k / d)
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * pos[:, None, None] * inv)
    np.testing.assert_allclose(y[..., : d // 2], z.real, rtol=0, atol=1e-9)
    np.testing.assert_allclose(y[..., d // 2:], z.imag, rtol=0, atol=1e-9)


def test_rope_frequencies_closed_form():
    """d = 4, theta = 1e4: pair 0 turns at 1 rad per position, pair 1 at 0.01."""
    x = np.zeros((2, 1, 4))
    x[0, 0, 0] = 1.0      # pair (0, 2)
    x[1, 0, 1] = 1.0      # pair (1, 3)
    y = oracle.rope_exact(x, np.array([3, 100]), 1e4, 1.0)
    np.testing.assert_allclose(y[0, 0], [math.cos(3), 0, math.sin(3), 0], atol=1e-12)
    np.testing.assert_allclose(y[1, 0], [0, math.cos(1), 0, math.sin(1)], atol=1e-12)
    # rope_scale multiplies the position
    y2 = oracle.rope_exact(x, np.array([6, 200]), 1e4, 0.5)
    np.testing.assert_allclose(y2, y, atol=1e-12)


def test_rope_norm_and_identity():
    w = make_custom_tree(17, [50], h_q=2, h_kv=2, d=128, dtype="bf16")
    x = w.q.double().numpy()
    pos = np.arange(50) * 37
    y = oracle.rope_exact(x, pos, 1e4, 1.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
    np.testing.assert_array_equal(oracle.rope(x, np.zeros(50, int), 1e4, 1.0, "bf16"), x)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_rope_rounded_within_half_ulp(dtype):
    w = make_custom_tree(18, [64], h_q=2, h_kv=2, d=64, dtype=dtype)
    pos = np.arange(64) * 61
    y = oracle.rope(w.q, pos, 1e4, 1.0, dtype)
    ye = oracle.rope_exact(w.q, pos, 1e4, 1.0)
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    # values are representable in dtype
    np.testing.assert_array_equal(torch.from_numpy(y).to(tdt).double().numpy(), y)
    eps = 2.0 ** (-11 if dtype == "f16" else -8)
    assert np.all(np.abs(y - ye) <= eps * np.maximum(np.abs(ye), 2.0 ** -14) * 1.01 + 1e-6)


def test_rope_relative_position_invariance():
    """Scores depend only on position differences: shifting every position by
    a constant moves out/lse only by the rounding of the rotated values."""
    w = make_custom_tree(19, [40, 17], h_q=4, h_kv=2, d=128, dtype="f16", rotary_mode=1,
                         max_children=3)
    out, lse = _tree_oracle(w)
    w.q_rope_position = w.q_rope_position + 1000
    out2, lse2 = _tree_oracle(w)
    assert np.abs(out - out2).max() < 2e-2
    assert np.abs(lse - lse2).max() < 2e-2
    # and exactly, before rounding:
    x = w.q.double().numpy()[:8]
    kk = w.k.double().numpy()[:8]
    p = np.arange(8)
    s1 = np.einsum("nhd,nhd->nh", oracle.rope_exact(x[:, :2], p, 1e4, 1.0), oracle.rope_exact(kk, p[::-1], 1e4, 1.0))
    s2 = np.einsum("nhd,nhd->nh", oracle.rope_exact(x[:, :2], p + 777, 1e4, 1.0), oracle.rope_exact(kk, p[::-1] + 777, 1e4, 1.0))
    np.testing.assert_allclose(s1, s2, atol=1e-9)


# ---------------------------------------------------------------------------
# paged KV
# ---------------------------------------------------------------------------

def test_page_permutation_invariance():
    w = make_custom_paged(20, [33, 7], [90, 40], h_q=4, h_kv=2, d=64, dtype="bf16", causal=1, extra_pages=5)
    pages = pages_from_logical(w)
    out, lse = _paged_oracle(w, pages=pages)
    perm = np.random.default_rng(3).permutation(w.num_pages)
    inv = np.argsort(perm)
    pages2 = pages[torch.from_numpy(inv)]            # new page i holds old page inv[i]
    w.page_values = perm[w.page_values].astype(np.int32)  # old page p is now at perm[p]
    out2, lse2 = _paged_oracle(w, pages=pages2)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_paged_tree_equals_contiguous_tree():
    """A paged tree with no prefix equals the contiguous tree operator."""
    w = make_custom_paged(21, [13, 30], [13, 30], h_q=4, h_kv=2, d=64, dtype="f16", causal=0, tree=True,
                          tree_max_children=3)
    out, lse = _paged_oracle(w)
    ip = w.q_indptr
    out2, lse2 = oracle.tree_attn(w.q, ip, w.k_store, w.v_store, ip, None, w.tree_order_indptr,
                                  w.tree_order, 0, 1.0, 1e4, w.sm_scale, w.dtype)
    np.testing.assert_allclose(out, out2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-12)


def test_sliding_window_equals_causal_on_sink_plus_window():
    stored, window, sink = [200, 77], [64, 40], [4, 0]
    qo = [20, 9]
    w = make_custom_paged(22, qo, stored, h_q=4, h_kv=2, d=64, dtype="bf16", causal=1,
                          sliding=([s - wd for s, wd in zip(stored, window)], sink))
    out, lse = _paged_oracle(w)
    for b in range(2):
        q0, q1 = int(w.q_indptr[b]), int(w.q_indptr[b + 1])
        s0 = int(w.kv_store_indptr[b])
        ks = torch.cat([w.k_store[s0:s0 + sink[b]], w.k_store[s0 + stored[b] - window[b]: s0 + stored[b]]])
        vs = torch.cat([w.v_store[s0:s0 + sink[b]], w.v_store[s0 + stored[b] - window[b]: s0 + stored[b]]])
        L = sink[b] + window[b]
        mask = torch.ones(q1 - q0, L, dtype=torch.bool).tril(diagonal=L - (q1 - q0)).numpy()
        ref = _sdpa(w.q[q0:q1].double(), _expand_kv(ks.double(), 2), _expand_kv(vs.double(), 2), mask, w.sm_scale)
        np.testing.assert_allclose(out[q0:q1], ref, rtol=0, atol=1e-10)


def test_cache_rope_equals_prerotated_pages():
    """K rotated before caching (oracle applies it after the gather) equals a
    cache whose pages already hold the rotated K."""
    w = make_custom_paged(23, [12, 20], [40, 20], h_q=4, h_kv=2, d=64, dtype="bf16", causal=1,
                          store_rope="linear", rope_theta=1e4)
    out, lse = _paged_oracle(w)
    kr = oracle.rope(w.k_store, w.store_rope_position, 1e4, 1.0, "bf16")
    w2_k = torch.from_numpy(kr).to(torch.bfloat16)
    w.k_store, w.store_rope_position = w2_k, None
    out2, lse2 = _paged_oracle(w)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_inkernel_k_rope_equals_cache_rope_at_offset():
    """In-kernel K rotation at k_rope_pos_offset[b] + j equals K rotated before
    caching at the same positions."""
    w = make_custom_paged(24, [8, 15], [30, 15], h_q=4, h_kv=2, d=64, dtype="f16", causal=1,
                          rotary_mode=1, k_rope_pos_offset=[5, 100])
    out, lse = _paged_oracle(w)
    w.store_rope_position = np.concatenate([np.arange(30) + 5, np.arange(15) + 100]).astype(np.int32)
    w.k_rope_pos_offset = None
    out2, lse2 = _paged_oracle(w)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


# ---------------------------------------------------------------------------
# degenerate cases (readings where the pages are silent)
# ---------------------------------------------------------------------------

def test_empty_rows_and_sequences():
    # kv shorter than qo: the first causal rows see nothing; seq 1 owns no pages
    w = make_custom_paged(25, [6, 3, 0], [4, 0, 5], h_q=2, h_kv=1, d=64, dtype="bf16", causal=1)
    out, lse = _paged_oracle(w)
    assert np.all(out[0:2] == 0) and np.all(np.isneginf(lse[0:2]))
    assert np.all(np.isfinite(lse[2:6]))
    assert np.all(out[6:9] == 0) and np.all(np.isneginf(lse[6:9]))


# ---------------------------------------------------------------------------
# brute force on the tiny workload
# ---------------------------------------------------------------------------

def test_scalar_bruteforce_agrees_on_tree_tiny():
    w = make_config(0)
    out, lse = _tree_oracle(w)
    q = w.q.double().tolist()
    k = w.k.double().tolist()
    v = w.v.double().tolist()
    so, sl = scalar.tree_attn_bruteforce(q, k, v, w.q_indptr, w.parents, w.h_q, w.h_kv, w.sm_scale)
    np.testing.assert_allclose(out, np.array(so), rtol=0, atol=1e-9)
    np.testing.assert_allclose(lse, np.array(sl), rtol=0, atol=1e-9)


def test_row_sampling_matches_full():
    w = make_custom_paged(26, [40, 25], [60, 25], h_q=4, h_kv=2, d=64, dtype="bf16", causal=1)
    out, lse = _paged_oracle(w)
    rows = np.array([0, 17, 39, 40, 64])
    out2, lse2 = _paged_oracle(w, rows=rows)
    np.testing.assert_array_equal(out[rows], out2[rows])
    others = np.setdiff1d(np.arange(w.total_q), rows)
    assert np.isnan(out2[others]).all()


# ---------------------------------------------------------------------------
# merge of states over disjoint key sets (split-KV)
# ---------------------------------------------------------------------------

def test_merge_of_split_key_sets_equals_attention_over_the_union():
    """Attention over a key set equals the merge of attention over any
    partition of it (pinned against the unsplit definition, which the other
    pins tie to SDPA); empty parts and fully empty rows included."""
    rng = np.random.default_rng(7)
    R, L, D = 6, 40, 16
    q = rng.standard_normal((R, D)); k = rng.standard_normal((L, D)); v = rng.standard_normal((L, D))
    vis = rng.random((R, L)) < 0.6
    vis[3] = False                      # no visible key at all
    vis[4, :] = False; vis[4, 35] = True   # one key, in the last part
    ref_o, ref_l = oracle.attend(q, k, v, vis, 0.3)
    cuts = [0, 7, 7, 20, 33, 40]        # includes an empty part
    parts = [oracle.attend(q, k[a:b], v[a:b], vis[:, a:b], 0.3) for a, b in zip(cuts[:-1], cuts[1:])]
    po = np.stack([p[0] for p in parts]); pl = np.stack([p[1] for p in parts])
    o, l = oracle.merge_states(po, pl)
    assert np.isneginf(l[3]) and np.all(o[3] == 0)
    np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-12)
    fin = np.isfinite(ref_l)
    np.testing.assert_allclose(l[fin], ref_l[fin], rtol=0, atol=1e-12)
    # a single part is the identity
    o1, l1 = oracle.merge_states(ref_o[None], ref_l[None])
    np.testing.assert_array_equal(o1, ref_o)


def test_merge_two_equal_halves_closed_form():
    """Two parts with equal lse: lse + 1 (base 2) and the mean of the outputs."""
    po = np.array([[[1.0, -2.0]], [[3.0, 4.0]]])
    pl = np.array([[0.5], [0.5]])
    o, l = oracle.merge_states(po, pl)
    np.testing.assert_allclose(l, [1.5], atol=1e-15)
    np.testing.assert_allclose(o, [[2.0, 1.0]], atol=1e-15)


# ---------------------------------------------------------------------------
# padded-batch masks (ragged prefill over contiguous K/V)
# ---------------------------------------------------------------------------

def _ragged(seed, qo, kv, h_q=4, h_kv=2, d=16):
    rng = np.random.default_rng(seed)
    q = torch.from_numpy(rng.standard_normal((sum(qo), h_q, d))).to(torch.float16)
    k = torch.from_numpy(rng.standard_normal((sum(kv), h_kv, d))).to(torch.float16)
    v = torch.from_numpy(rng.standard_normal((sum(kv), h_kv, d))).to(torch.float16)
    return q, np.concatenate([[0], np.cumsum(qo)]), k, v, np.concatenate([[0], np.cumsum(kv)])


def test_right_padding_equals_attention_on_the_valid_prefix():
    qo, kv, valid = [9, 12, 5], [9, 12, 7], [6, 12, 0]
    q, qi, k, v, ki = _ragged(50, qo, kv)
    out, lse = oracle.ragged_prefill(q, qi, k, v, ki, np.array(valid), 1, 0, 0.4)
    for b in range(3):
        n = valid[b]
        if n:
            ro, rl = oracle.ragged_prefill(q[qi[b]:qi[b] + n], np.array([0, n]), k[ki[b]:ki[b] + n],
                                           v[ki[b]:ki[b] + n], np.array([0, n]), None, 0, 0, 0.4)
            np.testing.assert_allclose(out[qi[b]:qi[b] + n], ro, atol=1e-12)
            np.testing.assert_allclose(lse[qi[b]:qi[b] + n], rl, atol=1e-12)
        # padding rows see nothing
        assert np.all(np.isneginf(lse[qi[b] + n:qi[b + 1]])) and np.all(out[qi[b] + n:qi[b + 1]] == 0)


def test_left_padding_equals_causal_attention_on_the_valid_suffix():
    qo, kv, valid = [8, 11, 4], [13, 11, 6], [5, 11, 0]
    q, qi, k, v, ki = _ragged(51, qo, kv)
    out, lse = oracle.ragged_prefill(q, qi, k, v, ki, np.array(valid), 2, 1, 0.4)
    for b in range(3):
        n = valid[b]
        pq, pk = qo[b] - n, kv[b] - n
        if n:
            sq, sk = slice(qi[b] + pq, qi[b + 1]), slice(ki[b] + pk, ki[b + 1])
            ro, rl = oracle.ragged_prefill(q[sq], np.array([0, n]), k[sk], v[sk], np.array([0, n]),
                                           None, 0, 1, 0.4)
            np.testing.assert_allclose(out[sq], ro, atol=1e-12)
            np.testing.assert_allclose(lse[sq], rl, atol=1e-12)
        assert np.all(np.isneginf(lse[qi[b]:qi[b] + pq])) and np.all(out[qi[b]:qi[b] + pq] == 0)


def test_plain_ragged_prefill_matches_paged_causal():
    """pad_mode 0 over contiguous K/V equals the paged causal path on the
    same rows (two independent gathers of the same definition)."""
    w = make_custom_paged(52, [7, 20], [30, 20], h_q=4, h_kv=2, d=16, dtype="f16", causal=1)
    po, pl = oracle.paged_attn(w.q, w.q_indptr, pages_from_logical(w), w.page_indptr, w.page_values,
                               w.length_info, 0, 1, w.sm_scale, w.dtype)
    k = torch.cat([w.k_store[int(w.kv_store_indptr[b]):int(w.kv_store_indptr[b + 1])] for b in range(2)])
    v = torch.cat([w.v_store[int(w.kv_store_indptr[b]):int(w.kv_store_indptr[b + 1])] for b in range(2)])
    ro, rl = oracle.ragged_prefill(w.q, w.q_indptr, k, v, w.kv_store_indptr, None, 0, 1, w.sm_scale)
    np.testing.assert_allclose(ro, po, atol=1e-12)
    np.testing.assert_allclose(rl, pl, atol=1e-12)


# ---------------------------------------------------------------------------
# multi-head latent attention over a latent page pool
# ---------------------------------------------------------------------------

def _mla(seed, qo, stored, h_q=4, d_qk=24, d_latent=16, causal=1, **kw):
    from workloads import make_custom_mla
    return make_custom_mla(seed, qo, stored, h_q=h_q, d_qk=d_qk, d_latent=d_latent, dtype="bf16",
                           causal=causal, **kw)


def _mla_oracle(w, pages=None, **kw):
    from workloads import mla_pages_from_logical
    pages = mla_pages_from_logical(w) if pages is None else pages
    return oracle.mla_paged_attn(w.q, w.q_indptr, pages, w.page_indptr, w.page_values, w.length_info,
                                 w.causal, w.sm_scale, w.d_latent, **kw)


@pytest.mark.parametrize("causal", [1, 0])
def test_mla_matches_sdpa_on_expanded_heads(causal):
    """Every query head reads the same latent rows: K = all d_qk columns,
    V = the first d_latent. Against torch SDPA on K/V replicated per head,
    with an explicit bottom-right mask; lse against scipy's logsumexp."""
    w = _mla(70, [5, 17, 0, 9, 4], [20, 17, 3, 40, 2], causal=causal)   # last: more queries than keys
    out, lse = _mla_oracle(w)
    for b in range(w.batch):
        q0, q1 = int(w.q_indptr[b]), int(w.q_indptr[b + 1])
        s0, s1 = int(w.kv_store_indptr[b]), int(w.kv_store_indptr[b + 1])
        if q1 == q0:
            continue
        kv = w.k_store[s0:s1].double().numpy()
        L, qo = s1 - s0, q1 - q0
        r = np.arange(qo)[:, None]
        c = np.arange(L)[None, :]
        mask = (c < L - qo + r + 1) if causal else np.ones((qo, L), bool)
        q = w.q[q0:q1].double().numpy()
        has = mask.any(axis=1)
        kh = np.repeat(kv[:, None, :], w.h_q, axis=1)
        vh = np.repeat(kv[:, None, :w.d_latent], w.h_q, axis=1)
        ref = _sdpa(q[has], kh, vh, mask[has], w.sm_scale)
        assert np.allclose(out[q0:q1][has], ref, atol=1e-12, rtol=1e-12)
        assert np.all(out[q0:q1][~has] == 0) and np.all(np.isneginf(lse[q0:q1][~has]))
        s = w.sm_scale * np.einsum("rhd,ld->rhl", q, kv)
        s = np.where(mask[:, None, :], s, -np.inf)
        ref_lse = scipy.special.logsumexp(s[has], axis=-1) / math.log(2.0)
        assert np.allclose(lse[q0:q1][has], ref_lse, atol=1e-12, rtol=1e-12)


def test_mla_absorbed_equals_mha_with_up_projections():
    """Absorbing the per-head key up-projection into q and the value
    up-projection after the output gives ordinary attention over the
    up-projected heads: with K_h = [C W_K,h | K_rope], V_h = C W_V,h and
    q_h = [q_n,h | q_r,h], MLA over the latent rows [C | K_rope] with
    q'_h = [q_n,h W_K,h^T | q_r,h] returns out'_h, and out'_h W_V,h equals
    softmax(q_h K_h^T) V_h (float64, SDPA on the expanded heads)."""
    rng = np.random.default_rng(71)
    L, qo, h, dc, dr, dh, dv = 37, 11, 3, 16, 8, 12, 10
    C = rng.standard_normal((L, dc))
    K_rope = rng.standard_normal((L, dr))
    W_K = rng.standard_normal((h, dc, dh)) / 4
    W_V = rng.standard_normal((h, dc, dv)) / 4
    q_n = rng.standard_normal((qo, h, dh))
    q_r = rng.standard_normal((qo, h, dr))
    scale = 0.3
    mask = np.arange(L)[None, :] < (L - qo + np.arange(qo)[:, None] + 1)
    K = np.stack([np.concatenate([C @ W_K[i], K_rope], axis=1) for i in range(h)], axis=1)   # [L, h, dh+dr]
    V = np.stack([C @ W_V[i] for i in range(h)], axis=1)                                     # [L, h, dv]
    Q = np.concatenate([q_n, q_r], axis=2)
    ref = _sdpa(Q, K, V, mask, scale)
    # latent side: one page table over ceil(L / 16) pages in reverse order
    npg = (L + 15) // 16
    pages = torch.zeros((npg, 16, dc + dr), dtype=torch.float64)
    kv = torch.from_numpy(np.concatenate([C, K_rope], axis=1))
    order = np.arange(npg)[::-1].astype(np.int32)
    for t in range(L):
        pages[order[t // 16], t % 16] = kv[t]
    q_lat = np.concatenate([np.einsum("rhd,hcd->rhc", q_n, W_K), q_r], axis=2)
    out_lat, _ = oracle.mla_paged_attn(q_lat, np.array([0, qo]), pages, np.array([0, npg]), order,
                                       np.array([L - 16 * (npg - 1)]), 1, scale, dc)
    got = np.einsum("rhc,hcv->rhv", out_lat, W_V)
    assert np.allclose(got, ref, atol=1e-10, rtol=1e-10)


def test_mla_single_visible_key_gives_latent_row():
    """Causal with no cached prefix: the first query token sees only key 0,
    so out = its first d_latent values and lse = s_0 / ln 2."""
    w = _mla(72, [6], [6])
    out, lse = _mla_oracle(w)
    kv0 = w.k_store[0].double().numpy()
    assert np.array_equal(out[0], np.broadcast_to(kv0[:w.d_latent], (w.h_q, w.d_latent)))
    s0 = w.sm_scale * w.q[0].double().numpy() @ kv0
    assert np.allclose(lse[0], s0 / math.log(2.0), atol=1e-12)


def test_mla_page_permutation_invariance():
    w = _mla(73, [9, 30], [40, 30], extra_pages=4)
    out1, lse1 = _mla_oracle(w)
    from workloads import mla_pages_from_logical
    pages = mla_pages_from_logical(w)
    perm = np.random.default_rng(5).permutation(w.num_pages)
    new_pages = torch.empty_like(pages)
    new_pages[torch.from_numpy(perm)] = pages
    w.page_values = perm[w.page_values].astype(np.int32)
    out2, lse2 = _mla_oracle(w, pages=new_pages)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)
