"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Small cases are compared element by element on every row; they span several
query tiles (128 or 256 packed rows) and 64-key KV tiles with ragged tails.
The five workloads run at their full sizes in the same launch configuration
the benchmark times: tree_tiny, tree_batched, paged_causal and paged_sliding
are compared on every row, spec_tree_paged on every fourth query token of
every sequence (offset by the sequence index, so every wave of every work
item is hit). Outputs are filled with NaN before each launch, so a row that
no work item writes fails the finiteness check on every row.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.parity import DeviceInputs, compare, run_oracle, say
from workloads import make_config, make_custom_paged, make_custom_ragged, make_custom_tree

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_ragged_gqa_amd as ra
    ra.library()


def _check(w, label, rows=None, ref=None, max_abs=None):
    say("[gpu] %s: launching (b=%d total_q=%d h=%d/%d d=%d %s)" % (label, w.batch, w.total_q, w.h_q, w.h_kv, w.d, w.dtype))
    di = DeviceInputs(w)
    di.poison()
    out, lse = di.launch()
    torch.cuda.synchronize()
    say("[gpu] %s: done" % label)
    # every row written (NaN-poisoned before the launch; no case here has a
    # row without visible keys except where the oracle says so)
    ref_out, ref_lse = run_oracle(w, rows=rows) if ref is None else ref
    d_out, d_lse = compare(out, lse, ref_out, ref_lse, rows=rows, label=label)
    if rows is not None:
        assert not torch.isnan(out).any().item(), "%s: rows left unwritten" % label
        assert not torch.isnan(lse).any().item(), "%s: lse rows left unwritten" % label
    n_rows = w.total_q if rows is None else len(rows)
    say("[gpu] %s: %d of %d query tokens compared (all heads): max|d out| %.2e  max rel|d lse| %.2e"
        % (label, n_rows, w.total_q, d_out, d_lse))
    if max_abs is not None:
        assert d_out <= max_abs, "%s: max |d out| %.3g above %g" % (label, d_out, max_abs)
    return di


# ---------------------------------------------------------------------------
# the five workloads at full size
# ---------------------------------------------------------------------------

_REF_CACHE = {}


def _config_rows(w, k):
    """Rows compared for workload k: all, except spec_tree_paged (every
    fourth token of each sequence, offset b mod 4)."""
    if k != 4:
        return None
    rows = [np.arange(int(w.q_indptr[b]) + b % 4, int(w.q_indptr[b + 1]), 4) for b in range(w.batch)]
    return np.concatenate(rows).astype(np.int64)


def _config_case(k):
    """(workload, rows, oracle result), the oracle computed once per module
    for the runs with both workgroup shapes."""
    if k not in _REF_CACHE:
        w = make_config(k)
        rows = _config_rows(w, k)
        say("[gpu] config%d: oracle on %s rows" % (k, "all" if rows is None else len(rows)))
        _REF_CACHE[k] = (w, rows, run_oracle(w, rows=rows))
    return _REF_CACHE[k]


@pytest.mark.parametrize("k", [0, 1, 2, 3, 4])
def test_config_parity(k):
    """The five workloads at full size; besides the per-element bound, every
    compared element within 1e-2 of the oracle outright."""
    w, rows, ref = _config_case(k)
    _check(w, "config%d %s" % (k, w.name), rows=rows, ref=ref, max_abs=1e-2)


# ---------------------------------------------------------------------------
# contiguous tree attention, small shapes
# ---------------------------------------------------------------------------

TREE_CASES = [
    dict(seed=1, sizes=[1, 37, 64, 300], h_q=32, h_kv=8, d=128, dtype="f16", rotary_mode=1, max_children=4),
    dict(seed=2, sizes=[5, 129, 250], h_q=6, h_kv=2, d=64, dtype="bf16", rotary_mode=0),
    dict(seed=3, sizes=[200], h_q=4, h_kv=4, d=64, dtype="f16", rotary_mode=1, position_offset=5000),
    dict(seed=4, sizes=[17, 90], h_q=16, h_kv=2, d=128, dtype="bf16", rotary_mode=1, rope_theta=5e5),
    dict(seed=5, sizes=[0, 3, 0, 65], h_q=8, h_kv=1, d=128, dtype="f16", rotary_mode=0),
    # one KV head for all query heads (g = 32: one token per wave)
    dict(seed=7, sizes=[33, 100], h_q=32, h_kv=1, d=64, dtype="f16", rotary_mode=1),
    # rope_scale and sm_scale away from their defaults
    dict(seed=8, sizes=[50, 130, 64], h_q=16, h_kv=4, d=128, dtype="bf16", rotary_mode=1,
         rope_scale=0.5, sm_scale=0.2, max_children=3, position_offset=900),
    dict(seed=9, sizes=[70], h_q=8, h_kv=2, d=64, dtype="f16", rotary_mode=0, sm_scale=0.03),
]


@pytest.mark.parametrize("case", range(len(TREE_CASES)))
def test_tree_small(case):
    c = dict(TREE_CASES[case])
    seed, sizes = c.pop("seed"), c.pop("sizes")
    w = make_custom_tree(seed, sizes, **c)
    _check(w, "tree_small[%d]" % case)


@pytest.mark.parametrize("h_q,h_kv,span", [(16, 4, None), (4, 4, None), (16, 4, 64), (16, 4, 65)])
def test_tree_rope_position_ranges(h_q, h_kv, span):
    """In-kernel RoPE on q and k with positions other than node depths. The
    kernel keeps one table row per position value when an item's query rows
    and first key tile span at most 64 positions; otherwise one row per token
    or key, or (one query head per KV head: 128 tokens per item) per-lane
    angles. span None: positions scattered over 300,000 values (the
    fallbacks); 64 and 65: every item's positions span exactly that many
    values (nodes 0 and 1 of each tree, in every item's first key tile, hold
    the smallest and largest)."""
    w = make_custom_tree(40, [90, 200], h_q=h_q, h_kv=h_kv, d=128, dtype="f16", rotary_mode=1,
                         max_children=4)
    rng = np.random.default_rng(41)
    if span is None:
        w.q_rope_position = rng.integers(0, 300000, size=w.total_q).astype(np.int32)
    else:
        pos = []
        for b in range(w.batch):
            n = int(w.q_indptr[b + 1] - w.q_indptr[b])
            base = 1000 * (b + 1)
            p = rng.integers(base, base + span, size=n)
            p[0], p[1] = base, base + span - 1
            pos.append(p)
        w.q_rope_position = np.concatenate(pos).astype(np.int32)
    _check(w, "tree_rope_positions[h%d/%d span %s]" % (h_q, h_kv, span))


def test_tree_chain_and_singletons():
    # a chain (causal) and a forest of singletons in one batch
    w = make_custom_tree(6, [70, 40], h_q=8, h_kv=2, d=128, dtype="bf16")
    w.tree_mask = np.concatenate([
        np.stack([np.arange(70), np.full(70, 70)], axis=1),          # chain: node i ancestor of all later
        np.stack([np.arange(40), np.arange(1, 41)], axis=1)]).astype(np.int32)
    di = _check(w, "tree_chain_singletons")
    # a node that sees only itself has the single weight 1: its output is its
    # own V row bit for bit (every singleton, and the chain's root)
    g = w.h_q // w.h_kv
    own = torch.cat([w.v[0:1], w.v[70:110]]).repeat_interleave(g, dim=1)
    got = torch.cat([di.out[0:1], di.out[70:110]]).cpu()
    assert torch.equal(got, own), "a one-key row differs from its V row"


# ---------------------------------------------------------------------------
# paged KV, small shapes
# ---------------------------------------------------------------------------

PAGED_CASES = [
    dict(seed=11, qo=[1, 100, 257, 3], stored=[1, 400, 288, 3], h_q=32, h_kv=8, d=128, dtype="bf16", causal=1, extra_pages=7),
    dict(seed=12, qo=[64, 33], stored=[64, 200], h_q=4, h_kv=2, d=64, dtype="f16", causal=1),
    dict(seed=13, qo=[50, 130], stored=[20, 130], h_q=8, h_kv=1, d=128, dtype="bf16", causal=1),   # kv < qo: empty rows
    dict(seed=14, qo=[40, 7], stored=[90, 200], h_q=64, h_kv=8, d=128, dtype="bf16", causal=0),
    dict(seed=15, qo=[0, 5, 0, 7], stored=[10, 0, 0, 30], h_q=6, h_kv=3, d=64, dtype="f16", causal=1),
    dict(seed=16, qo=[50, 10, 200], stored=[300, 64, 1000], h_q=64, h_kv=8, d=128, dtype="bf16", causal=1,
         sliding=([200, 0, 800], [4, 0, 16])),
    dict(seed=17, qo=[300], stored=[330], h_q=8, h_kv=8, d=128, dtype="bf16", causal=1,
         sliding=([100], [0])),                                                 # qo > chunk
    dict(seed=18, qo=[1, 40, 130], stored=[1, 117, 330], h_q=64, h_kv=8, d=128, dtype="bf16", causal=0,
         tree=True, tree_max_children=4, tree_max_depth=16, store_rope="tree", rotary_mode=1, rope_theta=5e5),
    dict(seed=19, qo=[20, 64], stored=[20, 96], h_q=8, h_kv=2, d=64, dtype="f16", causal=0, tree=True,
         tree_max_children=2),
    dict(seed=20, qo=[8, 15, 70], stored=[30, 15, 170], h_q=4, h_kv=2, d=64, dtype="f16", causal=1,
         rotary_mode=1, k_rope_pos_offset=[5, 100, 2000]),
    dict(seed=21, qo=[300, 44], stored=[900, 44], h_q=32, h_kv=8, d=128, dtype="bf16", causal=1,
         store_rope="linear", rope_theta=1e4),
    # sliding windows whose (offset - sink) is not a multiple of 16: the tile
    # grid is shifted by that remainder; sinks longer than one 16-row block
    dict(seed=22, qo=[33, 70], stored=[500, 260], h_q=8, h_kv=2, d=64, dtype="f16", causal=1,
         sliding=([321, 77], [21, 3])),
    dict(seed=23, qo=[5, 129, 64], stored=[777, 1000, 700], h_q=16, h_kv=4, d=128, dtype="bf16", causal=1,
         sliding=([511, 690, 650], [1, 7, 16])),
    # one KV head for all query heads: a token spans two waves (g = 64) or a
    # whole four-wave work item (g = 128)
    dict(seed=24, qo=[3, 70], stored=[500, 260], h_q=64, h_kv=1, d=128, dtype="bf16", causal=1,
         sliding=([300, 100], [4, 0])),
    dict(seed=25, qo=[5, 2, 9], stored=[100, 64, 9], h_q=128, h_kv=1, d=64, dtype="f16", causal=1),
    # rope_scale and sm_scale away from their defaults: in-kernel K rotation,
    # and a tree cache rotated when appended (mid-page appends)
    dict(seed=26, qo=[30, 100], stored=[200, 100], h_q=16, h_kv=4, d=128, dtype="bf16", causal=1,
         rotary_mode=1, k_rope_pos_offset=[7, 0], rope_scale=0.5, sm_scale=0.05),
    dict(seed=27, qo=[64, 200], stored=[301, 1000], h_q=32, h_kv=4, d=128, dtype="bf16", causal=0,
         tree=True, tree_max_children=4, tree_max_depth=16, store_rope="tree", rotary_mode=1,
         rope_theta=5e5, rope_scale=0.25, sm_scale=0.15),
    dict(seed=28, qo=[77, 5], stored=[500, 333], h_q=8, h_kv=2, d=64, dtype="f16", causal=1,
         store_rope="linear", rope_scale=0.5, sm_scale=0.3, sliding=None),
    # in-kernel K rotation with a tree mask, and with a sliding window + sink
    # (K at chunk position j rotated at k_rope_pos_offset[b] + j)
    dict(seed=29, qo=[40, 90], stored=[200, 90], h_q=16, h_kv=4, d=128, dtype="bf16", causal=0,
         tree=True, tree_max_children=3, rotary_mode=1, k_rope_pos_offset=[11, 3000]),
    dict(seed=30, qo=[20, 60], stored=[700, 300], h_q=8, h_kv=2, d=64, dtype="f16", causal=1,
         sliding=([500, 130], [4, 0]), rotary_mode=1, k_rope_pos_offset=[0, 77]),
]


@pytest.mark.parametrize("case", range(len(PAGED_CASES)))
def test_paged_small(case):
    c = dict(PAGED_CASES[case])
    seed, qo, stored = c.pop("seed"), c.pop("qo"), c.pop("stored")
    w = make_custom_paged(seed, qo, stored, **c)
    _check(w, "paged_small[%d]" % case)


# ---------------------------------------------------------------------------
# append (RoPE before caching), determinism, streams
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64)])
def test_append_matches_oracle_rope(dtype, d):
    import attention_ragged_gqa_amd as ra
    from tests.parity import gpu_pages
    from workloads import pages_from_logical
    w = make_custom_paged(30, [5, 9], [70, 300], h_q=4, h_kv=2, d=d, dtype=dtype, causal=1,
                          store_rope="linear", rope_theta=5e5)
    w.store_rope_position = (w.store_rope_position * 13 + 7).astype(np.int32)   # large angles
    say("[gpu] append %s d=%d" % (dtype, d))
    pool = gpu_pages(w, "cuda:0")
    torch.cuda.synchronize()
    ref = pages_from_logical(w)
    kr = torch.from_numpy(oracle.rope(w.k_store, w.store_rope_position, 5e5, 1.0, dtype)).to(w.q.dtype)
    w.k_store = kr
    ref_rot = pages_from_logical(w)
    got = pool.cpu()
    assert torch.equal(got[:, 1], ref[:, 1])                 # V copied bit-exactly
    # rotated K bit-identical: cos/sin correctly rounded to float32 and both
    # products rounded before the sum, on both sides
    n_diff = int((got[:, 0] != ref_rot[:, 0]).sum())
    assert n_diff == 0, "%d rotated K values differ from the oracle" % n_diff


@pytest.mark.parametrize("h_kv,d,batch", [(3, 128, 6), (1, 64, 9), (40, 128, 5), (64, 64, 3), (2, 128, 1500)])
def test_append_shapes(h_kv, d, batch):
    """The append kernel's token-to-workgroup shapes (a thread per 16-byte
    chunk pair, 256 threads): several tokens per workgroup with a pair count
    that does not divide it (h_kv 3, d 128: ten tokens of 24 pairs), many
    (h_kv 1, d 64: 64 tokens), one token of exactly 256 pairs (h_kv 64, d 64),
    one wider than the workgroup (h_kv 40, d 128: 320 pairs, looped over),
    and a batch of 1,500 sequences whose index arrays do not fit the LDS copy
    (searched in global memory). Prefix appended, then the new tokens
    mid-page; the whole pool against the oracle's rotation, bit-identical,
    unused slots zero."""
    from tests.parity import gpu_pages
    from workloads import pages_from_logical
    rng = np.random.default_rng(9900 + h_kv)
    qo = [int(x) for x in rng.integers(1, 40 if batch < 100 else 4, size=batch)]
    stored = [q + int(rng.integers(0, 70 if batch < 100 else 30)) for q in qo]
    w = make_custom_paged(9900 + h_kv, qo, stored, h_q=h_kv, h_kv=h_kv, d=d, dtype="bf16", causal=1,
                          store_rope="linear", rope_theta=1e4)
    say("[gpu] append shapes h_kv=%d d=%d batch=%d: %d tokens" % (h_kv, d, batch, sum(stored)))
    pool = gpu_pages(w, "cuda:0")
    torch.cuda.synchronize()
    ref = pages_from_logical(w)
    w.k_store = torch.from_numpy(oracle.rope(w.k_store, w.store_rope_position, 1e4, 1.0, "bf16")).to(w.q.dtype)
    ref_rot = pages_from_logical(w)
    got = pool.cpu()
    assert torch.equal(got[:, 1], ref[:, 1]), "V"
    n_diff = int((got[:, 0] != ref_rot[:, 0]).sum())
    assert n_diff == 0, "%d rotated K values differ from the oracle" % n_diff


@pytest.mark.parametrize("h_kv,d,dtype", [(2, 128, "bf16"), (3, 64, "f16"), (40, 128, "bf16")])
def test_append_without_rotation(h_kv, d, dtype):
    """rope_position NULL: K and V copied as they are. Prefix, then the new
    tokens mid-page, in two calls; the whole pool equals the pages built
    on the host from the same tokens, bit for bit (unused slots zero)."""
    from workloads import pages_from_logical
    import attention_ragged_gqa_amd as ra
    w = make_custom_paged(9990 + h_kv, [7, 30, 1], [40, 95, 17], h_q=h_kv, h_kv=h_kv, d=d, dtype=dtype,
                          causal=1)
    pool = torch.zeros((w.num_pages, 2, w.h_kv, 16, w.d), dtype=w.q.dtype, device="cuda")
    stored = np.diff(w.kv_store_indptr).astype(np.int64)
    new = np.minimum(np.diff(w.q_indptr).astype(np.int64), stored)
    for starts, lens in ((np.zeros(w.batch, np.int64), stored - new), (stored - new, new)):
        idx = np.concatenate([np.arange(int(w.kv_store_indptr[b]) + starts[b],
                                        int(w.kv_store_indptr[b]) + starts[b] + lens[b])
                              for b in range(w.batch)]).astype(np.int64)
        sel = torch.from_numpy(idx)
        indptr = np.zeros(w.batch + 1, np.int64)
        indptr[1:] = np.cumsum(lens)
        i32 = lambda a: torch.as_tensor(np.ascontiguousarray(a), dtype=torch.int32, device="cuda")
        ra.ra_paged_kv_append(w.k_store[sel].cuda(), w.v_store[sel].cuda(), i32(indptr), i32(starts), None,
                              i32(w.page_indptr), i32(w.page_values), pool)
    torch.cuda.synchronize()
    assert torch.equal(pool.cpu(), pages_from_logical(w)), "unrotated append differs from the host pages"


def test_append_workload_full_size():
    """The benchmark's append step at full size: spec_tree_paged's 32,768 new
    tree tokens (K rotated at prefix + depth, theta 5e5) appended twice into
    its 2.3 GB paged cache, after the 4,096-token prefixes. Every new token's
    page slot against the oracle's rotation (bit-identical K, V copied
    exactly), and every other value of the pool unchanged."""
    from workloads.device import AppendInputs
    w = make_config(4)
    ai = AppendInputs(w)
    before = ai.pool.clone()
    say("[gpu] append workload: %d tokens into %d pages" % (ai.n_tokens, w.num_pages))
    ai.launch()
    ai.launch()
    torch.cuda.synchronize()
    pages, slots, idx = [], [], []
    for b in range(w.batch):
        off = ai.new_start[b] + np.arange(ai.new_len[b])
        pages.append(w.page_values[w.page_indptr[b] + off // 16])
        slots.append(off % 16)
        idx.append(int(w.kv_store_indptr[b]) + off)
    pg = torch.from_numpy(np.concatenate(pages).astype(np.int64)).cuda()
    sl = torch.from_numpy(np.concatenate(slots).astype(np.int64)).cuda()
    idx = np.concatenate(idx).astype(np.int64)
    got_k = ai.pool[pg, 0, :, sl, :].cpu()                  # [n, h_kv, d]
    got_v = ai.pool[pg, 1, :, sl, :].cpu()
    ref_k = torch.from_numpy(oracle.rope(w.k_store[idx], np.asarray(w.store_rope_position)[idx],
                                         w.rope_theta, w.rope_scale, w.dtype)).to(w.q.dtype)
    assert torch.equal(got_v, w.v_store[idx]), "V not copied exactly"
    n_diff = int((got_k != ref_k).sum())
    assert n_diff == 0, "%d of %d rotated K values differ from the oracle" % (n_diff, got_k.numel())
    before[pg, :, :, sl, :] = ai.pool[pg, :, :, sl, :]
    assert torch.equal(ai.pool, before), "values outside the new tokens' slots changed"
    del ai, before
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,d,theta,scale", [("bf16", 128, 5e5, 1.0), ("f16", 64, 1e4, 0.5)])
def test_rotation_bit_exact_at_scale(dtype, d, theta, scale):
    """Two million values rotated by the append kernel (positions up to
    300,000) against the oracle's rotation: bit-identical, the storage-type
    rounding ties included (about one value in 65,536 lies exactly on one)."""
    import attention_ragged_gqa_amd as ra
    n, h = 2048 * 128 // d, 8
    g = torch.Generator().manual_seed(77)
    k = torch.randn(n, h, d, generator=g).to(torch.bfloat16 if dtype == "bf16" else torch.float16)
    pos = torch.randint(0, 300000, (n,), generator=g, dtype=torch.int32)
    npages = (n + 15) // 16
    pages = torch.zeros(npages, 2, h, 16, d, dtype=k.dtype, device="cuda")
    say("[gpu] rotation at scale %s d=%d: %d values" % (dtype, d, k.numel()))
    ra.ra_paged_kv_append(k.cuda(), k.cuda(), torch.tensor([0, n], dtype=torch.int32, device="cuda"),
                          torch.zeros(1, dtype=torch.int32, device="cuda"), pos.cuda(),
                          torch.tensor([0, npages], dtype=torch.int32, device="cuda"),
                          torch.arange(npages, dtype=torch.int32, device="cuda"), pages,
                          rope_scale=scale, rope_theta=theta)
    torch.cuda.synchronize()
    got = pages[:, 0].permute(0, 2, 1, 3).reshape(npages * 16, h, d)[:n].cpu()
    ref = torch.from_numpy(oracle.rope(k, pos.numpy(), theta, scale, dtype)).to(k.dtype)
    n_diff = int((got != ref).sum())
    assert n_diff == 0, "%d of %d rotated values differ from the oracle" % (n_diff, k.numel())


def test_append_mid_page_into_partly_filled_cache():
    """Appends that start mid-page and cross page boundaries, into a cache
    already holding earlier tokens of each sequence (three calls per
    sequence, starts not multiples of 16, one sequence receiving nothing in
    the middle call); the whole pool must equal the oracle's rotation of
    the stored tokens, and slots never written must stay zero."""
    from tests.parity import append_range
    from workloads import pages_from_logical
    w = make_custom_paged(34, [3, 9, 40, 1], [70, 300, 41, 17], h_q=4, h_kv=2, d=128, dtype="bf16",
                          causal=1, store_rope="linear", rope_theta=1e4, rope_scale=0.5, extra_pages=3)
    stored = np.diff(w.kv_store_indptr)
    cut1 = np.array([7, 129, 0, 17])          # first call: [0, cut1)
    cut2 = np.array([45, 129, 33, 17])        # second: [cut1, cut2) (sequence 1 and 3: nothing)
    say("[gpu] append mid-page: stored %s, cuts %s / %s" % (stored.tolist(), cut1.tolist(), cut2.tolist()))
    pool = torch.zeros((w.num_pages, 2, w.h_kv, 16, w.d), dtype=w.q.dtype, device="cuda:0")
    append_range(pool, w, np.zeros(w.batch, np.int64), cut1, "cuda:0")
    append_range(pool, w, cut1, cut2 - cut1, "cuda:0")
    append_range(pool, w, cut2, stored - cut2, "cuda:0")
    torch.cuda.synchronize()
    ref_v = pages_from_logical(w)
    w.k_store = torch.from_numpy(oracle.rope(w.k_store, w.store_rope_position, w.rope_theta,
                                             w.rope_scale, w.dtype)).to(w.q.dtype)
    ref = pages_from_logical(w)
    got = pool.cpu()
    assert torch.equal(got[:, 1], ref_v[:, 1]), "V rows differ"
    n_diff = int((got[:, 0] != ref[:, 0]).sum())
    assert n_diff == 0, "%d rotated K values differ from the oracle" % n_diff
    # the extra pages and the slots past each sequence's end were never written
    unused = ref_v[:, 1].abs().sum(dim=(1, 3)) == 0                 # [pages, slot]
    assert int(unused.sum()) > 0
    assert not got.permute(0, 3, 1, 2, 4)[unused].any().item(), "a slot no token maps to was written"


def test_deterministic_and_side_stream():
    w = make_custom_paged(31, [200, 77], [700, 77], h_q=32, h_kv=8, d=128, dtype="bf16", causal=1)
    di = DeviceInputs(w)
    say("[gpu] determinism")
    out1, lse1 = di.launch()
    out1, lse1 = out1.clone(), lse1.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        di.out.zero_()
        out2, lse2 = di.launch(stream=s)
    s.synchronize()
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


@pytest.mark.parametrize("n_waves", [0, 8])
def test_graph_replay_matches_eager(n_waves, waves):
    """The benchmark times HIP-graph replays of the launch: every replay, with
    eager work and synchronizations in between, must give the eager result
    (with the per-launch workgroup shape, and with eight waves forced)."""
    waves(n_waves)
    for w in (make_config(1),
              make_custom_paged(32, [130, 9], [300, 40], h_q=16, h_kv=4, d=64, dtype="f16", causal=1)):
        di = DeviceInputs(w)
        say("[gpu] graph replay: %s" % w.name)
        out_e, lse_e = di.launch()
        out_e, lse_e = out_e.clone(), lse_e.clone()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            di.launch()
        for rep in range(4):
            di.out.fill_(7.0)
            di.lse.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(di.out, out_e) and torch.equal(di.lse, lse_e), "replay %d differs" % rep
            di.launch()          # eager work between replays
            torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# split-KV (few query rows over long KV) and the state merge
# ---------------------------------------------------------------------------

SPLIT_CASES = {
    "decode_causal_bf16": dict(seed=40, qo=[1, 3, 16, 1, 0], kv=[3000, 700, 5000, 64, 900], h_q=32,
                               h_kv=8, d=128, dtype="bf16", causal=1),
    "decode_noncausal_f16_d64": dict(seed=41, qo=[2, 5], kv=[1500, 2100], h_q=16, h_kv=2, d=64,
                                     dtype="f16", causal=0),
    "decode_sliding": dict(seed=42, qo=[4, 1], kv=[9000, 5000], h_q=16, h_kv=4, d=128, dtype="bf16",
                           causal=1, sliding=([9000 - 2048, 5000 - 1024], [4, 0])),
    "decode_tree": dict(seed=43, qo=[12, 30], kv=[1200, 800], h_q=16, h_kv=4, d=128, dtype="bf16",
                        causal=0, tree=True),
}


@pytest.mark.parametrize("case", sorted(SPLIT_CASES))
@pytest.mark.parametrize("splits", [2, 7, 0])
def test_split_kv_matches_oracle(case, splits):
    c = dict(SPLIT_CASES[case])
    seed, qo, kv = c.pop("seed"), c.pop("qo"), c.pop("kv")
    w = make_custom_paged(seed, qo, kv, **c)
    say("[gpu] split-KV %s splits=%d" % (case, splits))
    di = DeviceInputs(w)
    out, lse = di.launch(num_kv_splits=splits)
    torch.cuda.synchronize()
    ref_out, ref_lse = run_oracle(w)
    d_out, d_lse = compare(out, lse, ref_out, ref_lse, label="%s/%d" % (case, splits))
    say("[gpu] split-KV %s splits=%d: max|d out| %.2e max rel|d lse| %.2e" % (case, splits, d_out, d_lse))


def test_merge_states_matches_oracle():
    rng = np.random.default_rng(44)
    S, rows, d = 5, 300, 128
    po = rng.standard_normal((S, rows, d)).astype(np.float32)
    pl = (rng.standard_normal((S, rows)) * 4).astype(np.float32)
    pl[1, :40] = -np.inf                 # empty ranges
    pl[:, 50] = -np.inf                  # a row with no visible key anywhere
    import attention_ragged_gqa_amd as ra
    for dtype in (torch.bfloat16, torch.float16):
        out = torch.empty(rows, d, dtype=dtype, device="cuda")
        lse = torch.empty(rows, dtype=torch.float32, device="cuda")
        ra.ra_merge_states(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(), out, lse)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle.merge_states(po.astype(np.float64), pl.astype(np.float64))
        compare(out, lse, ref_o, ref_l, label="merge %s" % dtype)


def test_paged_decode_full_size_split():
    """The decode workload the benchmark times with split-KV, every row, both
    entry points."""
    from workloads import make_extra
    w = make_extra("paged_decode")
    ref_out, ref_lse = run_oracle(w)
    di = DeviceInputs(w)
    for splits in (None, 0):
        say("[gpu] paged_decode splits=%s" % splits)
        out, lse = di.launch() if splits is None else di.launch(num_kv_splits=splits)
        torch.cuda.synchronize()
        compare(out, lse, ref_out, ref_lse, label="paged_decode/%s" % splits)



def test_paged_long_context():
    """Long sequences: 64 and 33 new causal queries over 131,072 and 70,001
    cached tokens (8,192 and 4,376 permuted pages, 2,048 and 1,094 KV tiles),
    K rotated when cached, h 8/1 (all eight query heads on one KV head), bf16.
    Every row, through the plain entry point and split (the library's count
    and seven ranges); out and lse are NaN-poisoned before each launch."""
    w = make_custom_paged(9100, [64, 33], [131072, 70001], h_q=8, h_kv=1, d=128, dtype="bf16",
                          causal=1, store_rope="linear", rope_theta=5e5, name="long_context")
    ref_out, ref_lse = run_oracle(w)
    di = DeviceInputs(w)
    for splits in (None, 0, 7):
        say("[gpu] long context splits=%s" % splits)
        di.poison()
        out, lse = di.launch() if splits is None else di.launch(num_kv_splits=splits)
        torch.cuda.synchronize()
        d_out, d_lse = compare(out, lse, ref_out, ref_lse, label="long context/%s" % splits)
        say("[gpu] long context splits=%s: max|d out| %.2e max rel|d lse| %.2e" % (splits, d_out, d_lse))



def test_page_pool_beyond_4gib():
    """Every page of the pool past its first 4 GiB (page numbers shifted by
    65,537 pages of 64 KiB into a 4.3 GB pool): the append kernel fills the
    cache there (K rotated on the way in, prefix then new tokens, mid-page)
    and attention reads it, plain, split and with a tree mask. The oracle
    runs on the same tokens in a compact pool. Every row."""
    import copy
    for tree in (False, True):
        w = make_custom_paged(9810 + tree, [100, 37], [1000, 600], h_q=16, h_kv=8, d=128, dtype="bf16",
                              causal=0 if tree else 1, tree=tree, store_rope="tree" if tree else "linear",
                              rotary_mode=1, rope_theta=5e5, name="pool_beyond_4gib")
        ref_out, ref_lse = run_oracle(w)
        page_bytes = 2 * w.h_kv * 16 * w.d * 2
        off = (1 << 32) // page_bytes + 1
        wb = copy.copy(w)
        wb.page_values = w.page_values + np.int32(off)
        wb.num_pages = w.num_pages + off
        say("[gpu] pool beyond 4 GiB (tree %s): %d pages of %d bytes" % (tree, wb.num_pages, page_bytes))
        di = DeviceInputs(wb)
        assert di.pages.numel() * di.pages.element_size() > (1 << 32)
        for splits in (None, 0):
            di.poison()
            out, lse = di.launch() if splits is None else di.launch(num_kv_splits=splits)
            torch.cuda.synchronize()
            d_out, d_lse = compare(out, lse, ref_out, ref_lse, label="pool beyond 4 GiB/%s/%s" % (tree, splits))
            say("[gpu] pool beyond 4 GiB tree=%s splits=%s: max|d out| %.2e max rel|d lse| %.2e"
                % (tree, splits, d_out, d_lse))
        del di
        torch.cuda.empty_cache()


@pytest.mark.parametrize("kind", ["ragged", "tree"])
def test_contiguous_kv_beyond_4gib(kind):
    """Contiguous K/V whose every key row lies past the first 4 GiB of the K
    and V tensors (kv_indptr shifted by 2,097,153 rows of 2 KiB; 4.3 GB
    each): ragged causal prefill and tree attention, every row, against the
    oracle on the compact tensors."""
    if kind == "ragged":
        w = make_custom_ragged(9830, [60, 17], [700, 300], h_q=16, h_kv=8, d=128, dtype="bf16", causal=1,
                               name="kv_beyond_4gib")
    else:
        w = make_custom_tree(9831, [200, 65], h_q=16, h_kv=8, d=128, dtype="bf16", max_children=3,
                             name="kv_beyond_4gib")
    ref_out, ref_lse = run_oracle(w)
    di = DeviceInputs(w)
    row_bytes = w.h_kv * w.d * 2
    pad = (1 << 32) // row_bytes + 1
    for name in ("k", "v"):
        t = getattr(di, name)
        big = torch.zeros((pad + t.shape[0],) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)
        big[pad:] = t
        setattr(di, name, big)
    di.kv_indptr = di.kv_indptr + pad
    say("[gpu] contiguous %s K/V beyond 4 GiB: %d rows of %d bytes" % (kind, di.k.shape[0], row_bytes))
    di.poison()
    out, lse = di.launch()
    torch.cuda.synchronize()
    d_out, d_lse = compare(out, lse, ref_out, ref_lse, label="%s K/V beyond 4 GiB" % kind)
    say("[gpu] contiguous %s K/V beyond 4 GiB: max|d out| %.2e max rel|d lse| %.2e" % (kind, d_out, d_lse))
    del di
    torch.cuda.empty_cache()


def test_queries_and_outputs_beyond_4gib():
    """Q and out rows past their tensors' first 4 GiB: a leading sequence of
    262,145 tokens x 64 heads (16 KiB per token) over a single key pushes
    the compared sequences' rows past 4 GiB of Q (4.3 GB) and out. Ragged
    causal prefill; the compared rows against the oracle on the compact
    inputs. Under the bottom-right causal mask only the leading sequence's
    last token sees its key (out = its V row of ones, lse = 0 with q = 0);
    the others see none (out 0, lse -inf). All NaN-poisoned before."""
    w = make_custom_ragged(9840, [90, 33], [400, 33], h_q=64, h_kv=8, d=128, dtype="bf16", causal=1,
                           name="q_beyond_4gib")
    ref_out, ref_lse = run_oracle(w)
    di = DeviceInputs(w)
    tok_bytes = w.h_q * w.d * 2
    pad = (1 << 32) // tok_bytes + 1
    dev = di.q.device

    def grow(t, n_front, fill):
        big = torch.full((n_front + t.shape[0],) + tuple(t.shape[1:]), fill, dtype=t.dtype, device=dev)
        big[n_front:] = t
        return big

    di.q = grow(di.q, pad, 0.0)
    di.k = grow(di.k, 1, 0.0)
    di.v = grow(di.v, 1, 1.0)           # the leading sequence's one key
    di.out = grow(di.out, pad, float("nan"))
    di.lse = grow(di.lse, pad, float("nan"))
    di.q_indptr = torch.cat([torch.zeros(1, dtype=torch.int32, device=dev), di.q_indptr + pad])
    di.kv_indptr = torch.cat([torch.zeros(1, dtype=torch.int32, device=dev), di.kv_indptr + 1])
    say("[gpu] Q/out beyond 4 GiB: %d tokens of %d bytes" % (di.q.shape[0], tok_bytes))
    di.poison()
    out, lse = di.launch()
    torch.cuda.synchronize()
    assert torch.all(out[:pad - 1] == 0).item() and torch.all(lse[:pad - 1] == -float("inf")).item()
    assert torch.all(out[pad - 1] == 1).item() and torch.all(lse[pad - 1] == 0).item()
    d_out, d_lse = compare(out[pad:], lse[pad:], ref_out, ref_lse, label="Q/out beyond 4 GiB")
    say("[gpu] Q/out beyond 4 GiB: max|d out| %.2e max rel|d lse| %.2e" % (d_out, d_lse))
    del di, out, lse
    torch.cuda.empty_cache()


def test_paged_tree_long_prefix():
    """Speculative trees of 200 and 129 nodes (at most 4 children, depth at
    most 16) over 60,000- and 33,000-token paged prefixes, q rotated inline
    at prefix length + depth, K cached rotated, h 16/2, bf16: every row, plain
    and with the library's split count."""
    w = make_custom_paged(9300, [200, 129], [60200, 33129], h_q=16, h_kv=2, d=128, dtype="bf16",
                          causal=0, tree=True, tree_max_children=4, tree_max_depth=16,
                          store_rope="tree", rotary_mode=1, rope_theta=5e5, name="tree_long_prefix")
    ref_out, ref_lse = run_oracle(w)
    di = DeviceInputs(w)
    for splits in (None, 0):
        say("[gpu] tree long prefix splits=%s" % splits)
        di.poison()
        out, lse = di.launch() if splits is None else di.launch(num_kv_splits=splits)
        torch.cuda.synchronize()
        d_out, d_lse = compare(out, lse, ref_out, ref_lse, label="tree long prefix/%s" % splits)
        say("[gpu] tree long prefix splits=%s: max|d out| %.2e max rel|d lse| %.2e" % (splits, d_out, d_lse))


# ---------------------------------------------------------------------------
# ragged prefill over contiguous K/V, padded batches
# ---------------------------------------------------------------------------

RAGGED_CASES = {
    "causal_bf16_d128": dict(seed=60, qo=[300, 1, 0, 129], kv=[700, 1, 5, 129], h_q=32, h_kv=8,
                             d=128, dtype="bf16", causal=1),
    "full_f16_d64": dict(seed=61, qo=[77, 200], kv=[50, 333], h_q=8, h_kv=8, d=64, dtype="f16",
                         causal=0),
    "right_pad_bf16": dict(seed=62, qo=[256, 256, 256, 100], kv=[256, 256, 256, 300], h_q=16, h_kv=4,
                           d=128, dtype="bf16", causal=0, pad_mode=1, valid_lens=[100, 256, 0, 400]),
    "right_pad_f16_d64": dict(seed=63, qo=[130, 70], kv=[130, 90], h_q=8, h_kv=2, d=64, dtype="f16",
                              causal=0, pad_mode=1, valid_lens=[65, 1]),
    "left_pad_causal_bf16": dict(seed=64, qo=[256, 256, 256, 64], kv=[256, 256, 300, 64], h_q=16,
                                 h_kv=4, d=128, dtype="bf16", causal=1, pad_mode=2,
                                 valid_lens=[100, 256, 200, 0]),
    "left_pad_causal_f16_d64": dict(seed=65, qo=[190, 33], kv=[190, 40], h_q=8, h_kv=1, d=64,
                                    dtype="f16", causal=1, pad_mode=2, valid_lens=[129, 500]),
    "causal_f16_sm_scale": dict(seed=66, qo=[100, 257], kv=[150, 257], h_q=8, h_kv=2, d=128,
                                dtype="f16", causal=1, sm_scale=0.3),
}


@pytest.mark.parametrize("case", sorted(RAGGED_CASES))
def test_ragged_prefill_padded(case):
    from workloads import make_custom_ragged
    c = dict(RAGGED_CASES[case])
    w = make_custom_ragged(c.pop("seed"), c.pop("qo"), c.pop("kv"), **c)
    _check(w, "ragged %s" % case)


@pytest.mark.parametrize("waves", [0, 4, 8])
def test_large_deep_trees(waves):
    """Trees of 1,500 and 900 nodes with at most two children (deep, spanning
    24 and 15 KV tiles) over 500- and 100-token paged prefixes, q rotated
    inline at prefix length + depth and K cached rotated; and contiguous
    trees of 1,000 and 300 nodes with inline q/k RoPE. Every row, each
    workgroup shape."""
    import attention_ragged_gqa_amd as ra
    ra.ra_set_workgroup_waves(waves)
    try:
        _check(make_custom_paged(9600, [1500, 900], [2000, 1000], h_q=16, h_kv=4, d=128, dtype="bf16",
                                 causal=0, tree=True, tree_max_children=2, store_rope="tree",
                                 rotary_mode=1, rope_theta=5e5),
               "deep paged trees, waves %d" % waves)
        _check(make_custom_tree(9601, [1000, 300], h_q=16, h_kv=2, d=128, dtype="bf16", rotary_mode=1,
                                max_children=2),
               "deep contiguous trees, waves %d" % waves)
    finally:
        ra.ra_set_workgroup_waves(0)


@pytest.mark.parametrize("waves", [0, 8])
def test_many_sequences(waves):
    """Batches beyond the item search's 64-sequence rounds: 300 paged causal
    sequences of 0-5 queries over up to 125 keys (empty ones included) and
    200 contiguous trees of 1-11 nodes with inline q/k RoPE; every row, with
    the workgroup shape chosen per launch and with eight waves."""
    import attention_ragged_gqa_amd as ra
    rng = np.random.default_rng(9500)
    qo = [int(x) for x in rng.integers(0, 6, size=300)]
    stored = [q + int(rng.integers(0, 120)) for q in qo]
    sizes = [int(x) for x in np.random.default_rng(9501).integers(1, 12, size=200)]
    ra.ra_set_workgroup_waves(waves)
    try:
        _check(make_custom_paged(9500, qo, stored, h_q=8, h_kv=2, d=128, dtype="bf16", causal=1),
               "300 paged sequences, waves %d" % waves)
        _check(make_custom_tree(9501, sizes, h_q=8, h_kv=4, d=64, dtype="f16", rotary_mode=1),
               "200 trees, waves %d" % waves)
    finally:
        ra.ra_set_workgroup_waves(0)


@pytest.mark.parametrize("pad_mode", [0, 2])
def test_ragged_prefill_long_kv(pad_mode):
    """Contiguous K/V over long sequences: 100 and 37 causal queries over
    50,000 and 20,037 keys (782 and 314 KV tiles), h 32/4, bf16, plain or
    left-padded to valid lengths of 41,000 and 9,000; every row."""
    from workloads import make_custom_ragged
    kw = dict(pad_mode=2, valid_lens=[41000, 9000]) if pad_mode == 2 else {}
    w = make_custom_ragged(9400, [100, 37], [50000, 20037], h_q=32, h_kv=4, d=128, dtype="bf16",
                           causal=1, name="ragged_long_kv", **kw)
    _check(w, "ragged long KV pad_mode %d" % pad_mode)


def test_ragged_left_padded_workload():
    from workloads import make_extra
    w = make_extra("ragged_left_padded")
    _check(w, w.name)


def test_invariances_bit_exact():
    """Metamorphic checks, no oracle: a row's arithmetic (its tiles in order,
    tiles without a visible key adding exact zeros) does not depend on how
    rows are packed or where pages live, so these hold bit for bit. Paged
    causal bf16 with inline q RoPE over a cache rotated when appended:
    (a) GQA with g = 4 equals the same K/V replicated to g = 1;
    (b) a permuted page table over a permuted pool equals the original;
    (c) each sequence run on its own equals its rows of the batched run;
    (d) four-wave and eight-wave workgroups give the same bits."""
    import copy
    w = make_custom_paged(9960, [70, 130, 9], [300, 130, 500], h_q=8, h_kv=2, d=128, dtype="bf16",
                          causal=1, store_rope="linear", rotary_mode=1, rope_theta=1e4, name="invariance")
    di = DeviceInputs(w)
    out, lse = di.launch()
    torch.cuda.synchronize()
    out, lse = out.clone(), lse.clone()
    g = w.h_q // w.h_kv
    # (a) replicated K/V, one query head per KV head
    wr = copy.copy(w)
    wr.h_kv = w.h_q
    wr.k_store = w.k_store.repeat_interleave(g, dim=1)
    wr.v_store = w.v_store.repeat_interleave(g, dim=1)
    out_r, lse_r = DeviceInputs(wr).launch()
    torch.cuda.synchronize()
    assert torch.equal(out_r, out) and torch.equal(lse_r, lse), "GQA differs from replicated KV"
    # (b) pages moved: pool2[perm[p]] = pool[p], page_values2 = perm[page_values]
    perm = torch.from_numpy(np.random.default_rng(9961).permutation(w.num_pages)).cuda()
    di2 = DeviceInputs(w)
    pool2 = torch.empty_like(di2.pages)
    pool2[perm] = di2.pages
    di2.pages = pool2
    di2.page_values = perm[di2.page_values.long()].to(torch.int32)
    out_p, lse_p = di2.launch()
    torch.cuda.synchronize()
    assert torch.equal(out_p, out) and torch.equal(lse_p, lse), "page permutation changes the result"
    # (c) one sequence at a time
    for b in range(w.batch):
        q0, q1 = int(w.q_indptr[b]), int(w.q_indptr[b + 1])
        p0, p1 = int(w.page_indptr[b]), int(w.page_indptr[b + 1])
        dd = DeviceInputs(w)
        dd.q = di.q[q0:q1].contiguous()
        dd.q_indptr = torch.tensor([0, q1 - q0], dtype=torch.int32, device="cuda")
        dd.q_rope_position = di.q_rope_position[q0:q1].contiguous()
        dd.page_indptr = torch.tensor([0, p1 - p0], dtype=torch.int32, device="cuda")
        dd.page_values = di.page_values[p0:p1].contiguous()
        dd.length_info = di.length_info[b:b + 1].contiguous()
        dd.out = torch.empty_like(dd.out[q0:q1])
        dd.lse = torch.empty_like(dd.lse[q0:q1])
        o1, l1 = dd.launch()
        torch.cuda.synchronize()
        assert torch.equal(o1, out[q0:q1]) and torch.equal(l1, lse[q0:q1]), "sequence %d alone differs" % b
    # (d) both workgroup shapes
    import attention_ragged_gqa_amd as ra
    try:
        for n in (4, 8):
            ra.ra_set_workgroup_waves(n)
            o_n, l_n = di.launch()
            torch.cuda.synchronize()
            assert torch.equal(o_n, out) and torch.equal(l_n, lse), "%d waves differ" % n
    finally:
        ra.ra_set_workgroup_waves(0)
    say("[gpu] invariances: GQA = replicated KV, page permutation, per-sequence runs, "
        "workgroup shapes: bit-identical")


def test_invariances_across_entry_points():
    """Bit for bit, no oracle: (e) tree attention over chains (every node the
    child of the previous one) equals causal ragged prefill on the same
    q/k/v, the tree test and the causal bound selecting the same keys;
    (f) causal attention over contiguous K/V equals the paged entry point
    over the same tokens behind a permuted page table (fp16 and bf16)."""
    import attention_ragged_gqa_amd as ra
    for dtype in ("f16", "bf16"):
        # (e) chains of 150 and 77 nodes, d 64, h 8/2
        w = make_custom_tree(9970, [150, 77], h_q=8, h_kv=2, d=64, dtype=dtype, name="chains")
        w.tree_mask = np.concatenate([np.stack([np.arange(n), np.full(n, n)], axis=1)
                                      for n in (150, 77)]).astype(np.int32)
        di = DeviceInputs(w)
        out_t, lse_t = di.launch()
        out_c, lse_c = ra.ra_ragged_prefill(di.q, di.q_indptr, di.k, di.v, di.kv_indptr, causal=1,
                                            sm_scale=w.sm_scale)
        torch.cuda.synchronize()
        assert torch.equal(out_t, out_c) and torch.equal(lse_t, lse_c), "%s: chain tree != causal" % dtype
        # (f) the same tokens contiguous and paged, 60 and 200 queries over 333 and 200 keys
        wp = make_custom_paged(9971, [60, 200], [333, 200], h_q=16, h_kv=4, d=128, dtype=dtype, causal=1,
                               name="contiguous_vs_paged")
        dp = DeviceInputs(wp)
        out_p, lse_p = dp.launch()
        k = wp.k_store.cuda()
        v = wp.v_store.cuda()
        kv_indptr = torch.from_numpy(wp.kv_store_indptr.astype(np.int32)).cuda()
        out_r, lse_r = ra.ra_ragged_prefill(dp.q, dp.q_indptr, k, v, kv_indptr, causal=1, sm_scale=wp.sm_scale)
        torch.cuda.synchronize()
        assert torch.equal(out_p, out_r) and torch.equal(lse_p, lse_r), "%s: paged != contiguous" % dtype
    say("[gpu] invariances across entry points: chain tree = causal, paged = contiguous: bit-identical")


@pytest.mark.parametrize("kind,dtype,waves", [("ragged", "bf16", 0), ("ragged", "f16", 8),
                                               ("paged", "bf16", 0), ("paged", "bf16", 8)])
def test_uniform_scores_are_prefix_means(kind, dtype, waves):
    """All scores equal (q = 0): every weight is 1, so under the causal mask
    out[t] is the mean of the first lim_t V rows of the chunk, lim_t =
    L - qo + t + 1, and lse = log2(lim_t): a closed form from a float64
    cumulative sum, independent of the oracle. 130 and 70 queries over 1,000
    and 70 keys (ties in every row maximum, up to 1,000 equal weights)."""
    import attention_ragged_gqa_amd as ra
    if kind == "ragged":
        w = make_custom_ragged(9950, [130, 70], [1000, 70], h_q=8, h_kv=2, d=128, dtype=dtype, causal=1,
                               name="uniform_ragged")
        vs = [w.v[int(w.kv_indptr[b]):int(w.kv_indptr[b + 1])] for b in range(w.batch)]
    else:
        w = make_custom_paged(9951, [130, 70], [1000, 70], h_q=8, h_kv=2, d=128, dtype=dtype, causal=1,
                              name="uniform_paged")
        vs = [w.v_store[int(w.kv_store_indptr[b]):int(w.kv_store_indptr[b + 1])] for b in range(w.batch)]
    w.q.zero_()
    ra.ra_set_workgroup_waves(waves)
    try:
        di = DeviceInputs(w)
        di.poison()
        out, lse = di.launch()
        torch.cuda.synchronize()
    finally:
        ra.ra_set_workgroup_waves(0)
    out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
    g = w.h_q // w.h_kv
    for b in range(w.batch):
        q0, qo = int(w.q_indptr[b]), int(w.q_indptr[b + 1]) - int(w.q_indptr[b])
        vb = vs[b].double().numpy()                                   # [L, h_kv, d]
        L = vb.shape[0]
        csum = np.cumsum(vb, axis=0)
        lim = L - qo + np.arange(qo) + 1                              # >= 1 here
        ref = csum[lim - 1] / lim[:, None, None]                      # [qo, h_kv, d]
        ref = np.repeat(ref, g, axis=1)                               # query head h reads h // g
        tol = 2e-3 + np.abs(ref) * (2.0 ** -8 if dtype == "bf16" else 2.0 ** -11)
        err = np.abs(out[q0:q0 + qo] - ref)
        assert np.all(err <= tol), "seq %d: max |d out| %.3g" % (b, err.max())
        lse_ref = np.log2(lim.astype(np.float64))[:, None]
        assert np.allclose(lse[q0:q0 + qo], lse_ref, rtol=1e-6, atol=1e-6), "seq %d lse" % b
    say("[gpu] uniform scores %s %s waves %d: prefix means and log2 counts hold" % (kind, dtype, waves))


# ---------------------------------------------------------------------------
# the running softmax reference moving after the first tile
# ---------------------------------------------------------------------------

_LOG2E = 1.4426950408889634


def _reference_moves(w, slack=8.0, tile=64):
    """How often the kernel's running row maximum would move after a row's
    first visible 64-key tile: the kernel keeps its reference until a tile
    raises a row's maximum more than `slack` log2 units above it, and only
    then rescales O and l. Scores in float64 from the stored Q and K (no
    RoPE in these cases), visibility from the oracle's own mask functions,
    tiles on the chunk's key grid from key 0. Returns (rows that move at
    least once, moves in all, query rows x heads)."""
    rows_moved = n_moves = n_rows = 0
    g = w.h_q // w.h_kv
    for b in range(w.batch):
        q0, q1 = int(w.q_indptr[b]), int(w.q_indptr[b + 1])
        qo = q1 - q0
        if w.kind == "paged":
            kb = w.k_store[int(w.kv_store_indptr[b]):int(w.kv_store_indptr[b + 1])]
        else:
            kb = w.k[int(w.kv_indptr[b]):int(w.kv_indptr[b + 1])]
        kv = kb.shape[0]
        if qo == 0 or kv == 0:
            continue
        rows = np.arange(qo)
        if w.kind == "tree" or w.tree_order is not None:
            order = (w.tree_mask[int(w.mn_indptr[b]):int(w.mn_indptr[b + 1])] if w.kind == "tree" else
                     w.tree_order[int(w.tree_order_indptr[b]):int(w.tree_order_indptr[b + 1])])
            vis = oracle.tree_visible(order, rows, kv, qo)
        else:
            vis = oracle.causal_visible(rows, kv, qo, w.causal)
        qf, kf = w.q[q0:q1].double().numpy(), kb.double().numpy()
        nt = (kv + tile - 1) // tile
        for h in range(w.h_q):
            sc = np.where(vis, qf[:, h] @ kf[:, h // g].T * (w.sm_scale * _LOG2E), -np.inf)
            padded = np.full((qo, nt * tile), -np.inf)
            padded[:, :kv] = sc
            tmax = padded.reshape(qo, nt, tile).max(axis=2)
            ref = np.full(qo, -np.inf)
            cnt = np.zeros(qo, np.int64)
            for t in range(nt):
                up = tmax[:, t] > ref + slack
                cnt += up & np.isfinite(ref)
                ref = np.where(up, tmax[:, t], ref)
            rows_moved += int(np.sum(cnt > 0))
            n_moves += int(cnt.sum())
            n_rows += qo
    return rows_moved, n_moves, n_rows


def _scale_rows(x, idx, factors):
    for i, f in zip(idx, factors):
        x[i] = (x[i].float() * f).to(x.dtype)


def _outgrow_case(kind, dtype):
    """sm_scale 0.5 (scores spread over tens of log2 units) and a few late
    keys scaled by 2-8, so row maxima jump past the reference repeatedly."""
    if kind == "ragged_causal":
        w = make_custom_ragged(9700, [300, 129], [700, 129], h_q=8, h_kv=2, d=128, dtype=dtype, causal=1,
                               sm_scale=0.5, name="outgrow_ragged")
        _scale_rows(w.k, [200, 420, 640], [2, 4, 8])
    elif kind == "paged_causal":
        w = make_custom_paged(9701, [200, 64], [900, 300], h_q=16, h_kv=2, d=128, dtype=dtype, causal=1,
                              sm_scale=0.5, name="outgrow_paged")
        _scale_rows(w.k_store, [300, 560, 880, 1150], [2, 4, 8, 6])
    elif kind == "tree":
        w = make_custom_tree(9702, [400, 150], h_q=8, h_kv=2, d=128, dtype=dtype, max_children=2,
                             sm_scale=0.5, name="outgrow_tree")
        _scale_rows(w.k, [100, 200, 300, 520], [2, 4, 8, 6])
    else:   # paged tree over a prefix
        w = make_custom_paged(9703, [300, 90], [800, 200], h_q=8, h_kv=1, d=128, dtype=dtype, causal=0,
                              tree=True, tree_max_children=2, sm_scale=0.5, name="outgrow_paged_tree")
        _scale_rows(w.k_store, [150, 400, 650, 950], [2, 4, 8, 6])
    return w


@pytest.mark.parametrize("waves", [0, 8])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("kind", ["ragged_causal", "paged_causal", "tree", "paged_tree"])
def test_scores_outgrow_the_reference(kind, dtype, waves):
    """Every row against the oracle where the running reference moves after
    the first tile (O and l rescaled, several times for some rows): with N(0,1)
    inputs at sm_scale 1/sqrt(d) it never does in cases of this size."""
    import attention_ragged_gqa_amd as ra
    w = _outgrow_case(kind, dtype)
    moved, n_moves, n_rows = _reference_moves(w)
    say("[gpu] outgrow %s %s: reference moves on %d of %d rows (%d moves)" % (kind, dtype, moved, n_rows,
                                                                            n_moves))
    assert moved >= 200 and n_moves > moved, "the case no longer moves the reference"
    ra.ra_set_workgroup_waves(waves)
    try:
        _check(w, "outgrow %s %s waves %d" % (kind, dtype, waves))
    finally:
        ra.ra_set_workgroup_waves(0)


@pytest.mark.parametrize("splits", [3, 0])
@pytest.mark.parametrize("kind", ["paged_causal", "paged_tree"])
def test_split_kv_scores_outgrow_the_reference(kind, splits):
    """The same moving reference inside split-KV ranges (fp32 partial states
    merged by the second kernel), three splits and the automatic count."""
    w = _outgrow_case(kind, "bf16")
    di = DeviceInputs(w)
    di.poison()
    out, lse = di.launch(num_kv_splits=splits)
    torch.cuda.synchronize()
    ref_out, ref_lse = run_oracle(w)
    d_out, d_lse = compare(out, lse, ref_out, ref_lse, label="outgrow split %s/%d" % (kind, splits))
    say("[gpu] outgrow split-KV %s splits=%d: max|d out| %.2e max rel|d lse| %.2e" % (kind, splits, d_out, d_lse))


# ---------------------------------------------------------------------------
# the other workgroup shape on the same cases: small cases choose four waves
# by default and the large workloads eight, so each is rerun with the other
# ---------------------------------------------------------------------------

@pytest.fixture
def waves():
    import attention_ragged_gqa_amd as ra

    def set_(n):
        ra.ra_set_workgroup_waves(n)
    yield set_
    ra.ra_set_workgroup_waves(0)


@pytest.mark.parametrize("case", range(len(TREE_CASES)))
def test_tree_small_eight_waves(case, waves):
    waves(8)
    test_tree_small(case)


def test_tree_chain_and_singletons_eight_waves(waves):
    waves(8)
    test_tree_chain_and_singletons()


@pytest.mark.parametrize("case", range(len(PAGED_CASES)))
def test_paged_small_eight_waves(case, waves):
    waves(8)
    test_paged_small(case)


@pytest.mark.parametrize("case", sorted(RAGGED_CASES))
def test_ragged_prefill_padded_eight_waves(case, waves):
    waves(8)
    test_ragged_prefill_padded(case)


@pytest.mark.parametrize("k", [0, 1, 2, 3, 4])
def test_config_parity_other_shape(k, waves):
    """The five workloads with the workgroup shape their launch does not
    choose by default: eight waves for the two tree workloads, four for the
    three large ones."""
    waves(8 if k < 2 else 4)
    test_config_parity(k)
