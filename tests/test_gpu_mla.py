"""GPU parity of multi-head latent attention (C: ra_mla_paged_prefill)
against the CPU oracle, through the C ABI.

Small cases span several 128-row work items and 32-key tiles with ragged
tails, empty sequences, rows without visible keys, fp16 and bf16, one to 128
query heads; two cases make scores outgrow a row's first-tile reference by
more than the P type's range, which makes the kernel compute the item again
against the row maxima. The benchmark's latent workload is compared on every
second query token of each sequence (offset by the sequence index: every
wave of every work item is hit), every row checked for being written.
"""

import numpy as np
import pytest
import torch

from tests.parity import DeviceInputs, compare, run_oracle, say
from workloads import make_custom_mla, make_extra

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_ragged_gqa_amd as ra
    ra.library()


def _check(w, label, rows=None):
    say("[gpu] %s: launching (b=%d total_q=%d h_q=%d %s)" % (label, w.batch, w.total_q, w.h_q, w.dtype))
    di = DeviceInputs(w)
    di.poison()
    out, lse = di.launch()
    torch.cuda.synchronize()
    say("[gpu] %s: done" % label)
    ref_out, ref_lse = run_oracle(w, rows=rows)
    d_out, d_lse = compare(out, lse, ref_out, ref_lse, rows=rows, label=label)
    if rows is not None:
        assert not torch.isnan(out).any().item() and not torch.isnan(lse).any().item(), "rows left unwritten"
    say("[gpu] %s: %d of %d query tokens compared: max|d out| %.2e  max rel|d lse| %.2e"
        % (label, w.total_q if rows is None else len(rows), w.total_q, d_out, d_lse))


MLA_CASES = [
    dict(seed=90, qo=[1, 100, 257, 3], stored=[1, 400, 288, 3], h_q=16, dtype="bf16", causal=1, extra_pages=5),
    dict(seed=91, qo=[64, 33], stored=[64, 200], h_q=8, dtype="f16", causal=1),
    dict(seed=92, qo=[50, 130, 0], stored=[20, 130, 40], h_q=16, dtype="bf16", causal=1),   # kv < qo: empty rows
    dict(seed=93, qo=[40, 7], stored=[90, 200], h_q=128, dtype="bf16", causal=0),
    dict(seed=94, qo=[0, 5, 0, 7], stored=[10, 0, 0, 30], h_q=1, dtype="f16", causal=1),
    dict(seed=95, qo=[300], stored=[301], h_q=16, dtype="bf16", causal=1, sm_scale=0.02),
]


@pytest.mark.parametrize("case", range(len(MLA_CASES)))
def test_mla_small(case):
    c = dict(MLA_CASES[case])
    w = make_custom_mla(c.pop("seed"), c.pop("qo"), c.pop("stored"), d_qk=576, d_latent=512, **c)
    _check(w, "mla_small[%d]" % case)


def test_mla_long_context():
    """32 and 17 new causal queries over 40,000 and 65,536 cached latent rows
    (2,500 and 4,096 permuted pages, 1,250 and 2,048 KV tiles), 16 heads,
    bf16, every row."""
    w = make_custom_mla(9200, [32, 17], [40000, 65536], h_q=16, d_qk=576, d_latent=512, dtype="bf16",
                        causal=1, name="mla_long_context")
    _check(w, "mla long context")


def _outgrowing_rows(w, headroom):
    """Query rows (token, head) whose maximum score exceeds the maximum over
    their first 32 keys by more than `headroom` log2 units (the case the
    kernel recomputes); computed here in float64 from the inputs."""
    n = 0
    for b in range(w.batch):
        q0, q1 = int(w.q_indptr[b]), int(w.q_indptr[b + 1])
        s0, s1 = int(w.kv_store_indptr[b]), int(w.kv_store_indptr[b + 1])
        if q1 == q0 or s1 == s0:
            continue
        kv = w.k_store[s0:s1].double().numpy()
        sc = w.sm_scale / np.log(2.0) * np.einsum("thd,ld->thl", w.q[q0:q1].double().numpy(), kv)
        L, qo = s1 - s0, q1 - q0
        lim = np.minimum(L, L - qo + np.arange(qo) + 1) if w.causal else np.full(qo, L)
        for t in range(qo):
            if lim[t] <= 0:
                continue
            first = sc[t, :, :min(32, lim[t])].max(axis=-1)
            n += int(np.sum(sc[t, :, :lim[t]].max(axis=-1) > first + headroom))
    return n


def test_mla_scores_outgrow_the_first_tile_fp16():
    """fp16 P holds at most 2^15 above a row's reference: with sm_scale 0.3
    the scores spread over tens of log2 units, so many rows outgrow the
    maximum of their first tile."""
    w = make_custom_mla(96, [70, 129], [600, 400], h_q=8, d_qk=576, d_latent=512, dtype="f16",
                        causal=1, sm_scale=0.3)
    assert _outgrowing_rows(w, 15.0) > 0
    _check(w, "mla_outgrow_f16")


def test_mla_scores_outgrow_the_first_tile_bf16():
    """The rotary part (the last 64 values, which only K reads) of one late
    key of each sequence scaled by 150: many rows that see it score it far
    above anything in their first tile (more than the 64 log2 units bf16 P
    is allowed above the reference), while V keeps its N(0,1) values."""
    w = make_custom_mla(97, [40, 90], [500, 300], h_q=16, d_qk=576, d_latent=512, dtype="bf16",
                        causal=1)
    for b in range(w.batch):
        s1 = int(w.kv_store_indptr[b + 1])
        w.k_store[s1 - 5, 512:] = (w.k_store[s1 - 5, 512:].float() * 150).to(w.k_store.dtype)
    assert _outgrowing_rows(w, 64.0) > 0
    _check(w, "mla_outgrow_bf16")


def test_mla_prefill_workload():
    w = make_extra("mla_prefill")
    rows = np.concatenate([np.arange(int(w.q_indptr[b]) + b % 2, int(w.q_indptr[b + 1]), 2)
                           for b in range(w.batch)]).astype(np.int64)
    _check(w, "mla_prefill", rows=rows)


def test_mla_page_pool_beyond_4gib():
    """Every latent page past the pool's first 4 GiB (page numbers shifted by
    233,017 pages of 18 KiB into a 4.3 GB pool); the oracle reads the same
    rows from a compact pool. Every row."""
    w = make_custom_mla(9820, [80, 40], [700, 300], h_q=16, d_qk=576, d_latent=512, dtype="bf16", causal=1)
    ref = run_oracle(w)
    di = DeviceInputs(w)
    page_bytes = di.pages[0].numel() * di.pages.element_size()
    off = (1 << 32) // page_bytes + 1
    big = torch.zeros((off + di.pages.shape[0],) + tuple(di.pages.shape[1:]), dtype=di.pages.dtype,
                      device=di.pages.device)
    big[off:] = di.pages
    di.pages = big
    di.page_values = di.page_values + off
    assert big.numel() * big.element_size() > (1 << 32)
    say("[gpu] latent pool beyond 4 GiB: %d pages of %d bytes" % (big.shape[0], page_bytes))
    di.poison()
    out, lse = di.launch()
    torch.cuda.synchronize()
    d_out, d_lse = compare(out, lse, ref[0], ref[1], label="latent pool beyond 4 GiB")
    say("[gpu] latent pool beyond 4 GiB: max|d out| %.2e max rel|d lse| %.2e" % (d_out, d_lse))


def test_mla_invariances_bit_exact():
    """No oracle: a permuted page table over a permuted latent pool, and each
    sequence run on its own, give the batched run's bits (bf16, causal)."""
    import attention_ragged_gqa_amd as ra
    w = make_custom_mla(9980, [70, 129, 5], [300, 129, 400], h_q=16, d_qk=576, d_latent=512, dtype="bf16",
                        causal=1)
    di = DeviceInputs(w)
    out, lse = di.launch()
    torch.cuda.synchronize()
    out, lse = out.clone(), lse.clone()
    perm = torch.from_numpy(np.random.default_rng(9981).permutation(w.num_pages)).cuda()
    pool = torch.empty_like(di.pages)
    pool[perm] = di.pages
    o_p, l_p = ra.ra_mla_paged_prefill(di.q, di.q_indptr, pool, di.page_indptr,
                                       perm[di.page_values.long()].to(torch.int32), di.length_info,
                                       causal=1, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o_p, out) and torch.equal(l_p, lse), "page permutation changes the result"
    for b in range(w.batch):
        q0, q1 = int(w.q_indptr[b]), int(w.q_indptr[b + 1])
        p0, p1 = int(w.page_indptr[b]), int(w.page_indptr[b + 1])
        o1, l1 = ra.ra_mla_paged_prefill(di.q[q0:q1].contiguous(),
                                         torch.tensor([0, q1 - q0], dtype=torch.int32, device="cuda"),
                                         di.pages, torch.tensor([0, p1 - p0], dtype=torch.int32, device="cuda"),
                                         di.page_values[p0:p1].contiguous(), di.length_info[b:b + 1].contiguous(),
                                         causal=1, sm_scale=w.sm_scale)
        torch.cuda.synchronize()
        assert torch.equal(o1, out[q0:q1]) and torch.equal(l1, lse[q0:q1]), "sequence %d alone differs" % b
    say("[gpu] latent invariances: page permutation and per-sequence runs bit-identical")
