"""CPU checks of the benchmark's work accounting and of the parity tolerance.

bench.visible_pairs uses closed forms (tree depth + 1 ancestors, causal row
limits); here they are checked against the oracle's masks counted directly.
"""

import os
import numpy as np
import torch

import bench
import oracle
from tests.parity import out_tolerance
from workloads import make_config, make_custom_paged, make_custom_ragged, make_custom_tree


def _count_with_oracle(w, rows_only=False):
    """Visible (row, head, key) triples from the oracle's masks, or with
    rows_only the query tokens that see at least one key."""
    total = 0
    L = bench.chunk_lengths(w)
    for b in range(w.batch):
        q0, q1 = int(w.q_indptr[b]), int(w.q_indptr[b + 1])
        qo = q1 - q0
        if qo == 0:
            continue
        rows = np.arange(qo)
        if w.kind == "ragged":
            vis = oracle.padded_visible(rows, int(L[b]), qo, int(w.valid_len[b]) if w.pad_mode else 0,
                                        w.pad_mode, w.causal)
        elif w.kind == "tree":
            vis = oracle.tree_visible(w.tree_mask[int(w.mn_indptr[b]):int(w.mn_indptr[b + 1])], rows, int(L[b]), qo)
        elif w.tree_order is not None:
            t = w.tree_order[int(w.tree_order_indptr[b]):int(w.tree_order_indptr[b + 1])]
            vis = oracle.tree_visible(t, rows, int(L[b]), qo)
        else:
            vis = oracle.causal_visible(rows, int(L[b]), qo, w.causal)
        total += int(vis.any(axis=1).sum()) if rows_only else int(vis.sum())
    return total if rows_only else total * w.h_q


def _accounting_cases():
    return [
        make_config(0),
        make_config(1),
        make_custom_tree(1, [0, 5, 33], h_q=4, h_kv=2, d=64, dtype="f16", max_children=2),
        make_custom_paged(2, [7, 40, 0], [30, 40, 5], h_q=4, h_kv=1, d=64, dtype="bf16", causal=1),
        make_custom_paged(3, [7, 40], [30, 20], h_q=4, h_kv=1, d=64, dtype="bf16", causal=0),
        make_custom_paged(4, [20, 9], [200, 77], h_q=4, h_kv=2, d=64, dtype="bf16", causal=1,
                          sliding=([136, 37], [4, 0])),
        make_custom_paged(5, [6, 11], [26, 14], h_q=4, h_kv=2, d=64, dtype="f16", causal=0, tree=True),
        make_custom_ragged(6, [9, 12, 5], [9, 12, 7], h_q=4, h_kv=2, d=16, dtype="f16", causal=0,
                           pad_mode=1, valid_lens=[6, 15, 0]),
        make_custom_ragged(7, [8, 11, 4], [13, 11, 6], h_q=4, h_kv=2, d=16, dtype="f16", causal=1,
                           pad_mode=2, valid_lens=[5, 11, 0]),
        make_custom_ragged(8, [8, 20], [13, 20], h_q=4, h_kv=2, d=16, dtype="f16", causal=1),
        make_custom_ragged(9, [9, 6], [4, 6], h_q=4, h_kv=2, d=16, dtype="f16", causal=1),   # kv < qo
    ]


def test_visible_pairs_tree_and_causal():
    for w in _accounting_cases():
        assert bench.visible_pairs(w) == _count_with_oracle(w), w.name


def test_rows_with_keys_match_oracle_masks():
    """The Q bytes of the roofline count only rows that see a key (the
    kernels skip the others' Q); checked against the oracle's masks."""
    for w in _accounting_cases():
        assert bench.rows_with_keys(w) == _count_with_oracle(w, rows_only=True), w.name
    w = make_custom_ragged(7, [8, 11, 4], [13, 11, 6], h_q=4, h_kv=2, d=16, dtype="f16", causal=1,
                           pad_mode=2, valid_lens=[5, 11, 0])
    assert bench.rows_with_keys(w) == 5 + 11 + 0


def test_sliding_config_pairs_closed_form():
    w = make_config(3)
    # 4 sequences, chunk 4100, 1024 causal rows: row r sees 3077 + r columns
    assert bench.visible_pairs(w) == 4 * sum(3077 + r for r in range(1024)) * 64


def test_algorithmic_bytes_tree_batched():
    w = make_config(1)
    q = 1024 * 32 * 128 * 2
    kv = 1024 * 8 * 128 * 2 * 2
    lse = 1024 * 32 * 4
    idx = 4 * 17 * 2 + 4 * 17 + 8 * 1024 + 4 * 1024
    assert bench.algorithmic_bytes(w) == 2 * q + kv + lse + idx


def test_out_tolerance_only_relaxes_where_dtype_cannot_hold_1e2():
    bf, hf = torch.bfloat16, torch.float16
    assert np.all(out_tolerance(np.array([0.0, 0.3, 1.9, 3.99, -3.5]), bf) == 1e-2)
    assert np.all(out_tolerance(np.array([0.0, 5.0, 31.0]), hf) == 1e-2)
    assert abs(out_tolerance(np.array([5.0]), bf)[0] - (2.0 ** -6 + 2e-3)) < 1e-12
    assert abs(out_tolerance(np.array([-9.0]), bf)[0] - (2.0 ** -5 + 2e-3)) < 1e-12


def test_out_tolerance_weight_rounding_term():
    """With the oracle's spread sigma, the bound adds 2 u sigma (u = 2^-8 in
    bf16, 2^-11 in fp16), never going below 1e-2; a NaN spread (row not
    evaluated) adds nothing."""
    bf, hf = torch.bfloat16, torch.float16
    t = out_tolerance(np.array([2.0, 0.1, 2.0]), bf, np.array([1.0, 0.5, np.nan]))
    assert abs(t[0] - (2.0 ** -7 + 2e-3 + 2 * 2.0 ** -8 * 1.0)) < 1e-12
    assert t[1] == 1e-2 and abs(t[2] - 1e-2) < 1e-12
    t = out_tolerance(np.array([20.0]), hf, np.array([3.0]))
    assert abs(t[0] - max(1e-2, 2.0 ** -7 + 2e-3 + 2 * 2.0 ** -11 * 3.0)) < 1e-12


def test_visible_pairs_per_sequence_sum_to_total():
    for w in (make_config(1), make_custom_paged(9, [7, 40, 0, 3], [30, 40, 5, 80], h_q=4, h_kv=1, d=64,
                                                dtype="bf16", causal=1)):
        assert sum(bench.visible_pairs(w, seqs=[b]) for b in range(w.batch)) == bench.visible_pairs(w)


def test_cpu_baseline_counts_what_it_times():
    w = make_config(0)
    r = bench.cpu_baseline(w, bench.visible_pairs(w), budget_s=0.2)
    assert r["kind"] == "oracle" and r["value"] > 0 and r["cores"] >= 1
    assert r["host_cpus"] == os.cpu_count() and isinstance(r["cpu"], str)
    assert r["estimated"] is False
    w = make_custom_paged(10, [300, 200, 100], [400, 200, 900], h_q=128, h_kv=8, d=64, dtype="bf16",
                          causal=1)
    r = bench.cpu_baseline(w, bench.visible_pairs(w), budget_s=0.01)
    assert r["sample"].startswith("sequences 0..0 of 3")   # one whole sequence, then the budget is spent


def test_bound_of_configs():
    assert bench.bound_of(make_config(1)) == "hbm"
    assert bench.bound_of(make_config(2)) == "mfma"


def test_latent_attention_accounting():
    from workloads import make_custom_mla
    w = make_custom_mla(11, [5, 0, 7], [20, 4, 7], h_q=4, d_qk=576, d_latent=512, dtype="bf16", causal=1)
    # causal rows: sequence 0 sees 16..20 keys, sequence 2 sees 1..7
    pairs = (sum(range(16, 21)) + sum(range(1, 8))) * 4
    assert bench.visible_pairs(w) == pairs
    assert bench.flops_per_pair(w) == 2 * (576 + 512)
    q_out = 12 * 4 * (576 + 512) * 2 + 12 * 4 * 4
    kv = (20 + 7) * 576 * 2                     # one latent row per key of the sequences with queries
    idx = 4 * 4 * 2 + 4 * (2 + 1 + 1) + 4 * 3
    assert bench.algorithmic_bytes(w) == q_out + kv + idx


def test_kernel_hash_ignores_comments_only():
    """The hash that ties profiles/ to the kernel source skips comments and
    layout but not code or string literals."""
    a = 'int f() { // one\n  return 1; /* two */ }\nconst char* s = "// not a comment";\n'
    b = 'int f() {   // other words\n\n  return 1;   }\nconst char* s = "// not a comment";'
    c = 'int f() { return 2; }\nconst char* s = "// not a comment";\n'
    d = 'int f() { return 1; }\nconst char* s = "// changed";\n'
    assert bench.source_code_text(a) == bench.source_code_text(b)
    assert bench.source_code_text(a) != bench.source_code_text(c)
    assert bench.source_code_text(a) != bench.source_code_text(d)
    assert bench.kernel_source_hash("attn_fwd_kernel") != bench.kernel_source_hash("mla_fwd_kernel")


def test_timing_label_by_input_footprint():
    assert bench.timing_label({"copies": 26, "bytes": 21 << 20}) == "cold (26 input copies cycled)"
    assert bench.timing_label({"copies": 1, "bytes": 1 << 30}).startswith("one copy of 1024 MB, larger than")
    assert bench.timing_label({"copies": 1, "bytes": 100 << 20}) == "warm"


def test_append_bytes_closed_form():
    """Two sequences whose new tokens start mid-page: 5 tokens at storage
    offsets 15..19 (pages 0 and 1 of the sequence) and 17 at 23..39 (pages 1
    and 2). Each new token's K and V rows are read once and written once;
    int32 positions, append indptr (b + 1), starts (b), page indptr (b + 1)
    and the 4 page-table entries touched."""
    from types import SimpleNamespace
    w = make_custom_paged(5, [5, 17], [20, 40], h_q=4, h_kv=2, d=64, dtype="bf16", causal=1,
                          store_rope="linear")
    ai = SimpleNamespace(w=w, n_tokens=22, new_start=np.array([15, 23]), new_len=np.array([5, 17]))
    row = 2 * 64 * 2
    assert bench.append_bytes(ai) == 4 * 22 * row + 4 * 22 + 4 * 3 + 4 * 2 + 4 * 3 + 4 * 4
    assert bench.kernel_name(bench.APPEND_NAME) == "kv_append_kernel"
    assert bench.kernel_source_hash("kv_append_kernel") != bench.kernel_source_hash("attn_fwd_kernel")
