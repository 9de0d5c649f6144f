"""Helpers shared by the GPU parity tests: run a workload through the HIP
library (via the C ABI binding) and through the CPU oracle, and compare.

Tolerances (fp16/bf16 outputs against the float64 oracle):
  |out_gpu - out_ref| <= 1e-2 per element, except where the output dtype
    cannot hold the value that closely: storing a correct result rounds it by
    up to half an ulp, which for bf16 exceeds 1e-2 once |out| >= 4 (half-ulp
    0.0156 there). Such elements get half an ulp of |out_ref| plus 2e-3 for
    the arithmetic (P rounded to the MMA input type); for |out| < 4 in bf16
    and |out| < 32 in fp16 the bound stays exactly 1e-2.
  |lse_gpu - lse_ref| <= 1e-3 * max(1, |lse_ref|)
Rows with no visible key must be out == 0 and lse == -inf on both sides.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from workloads import pages_from_logical
from workloads.device import DeviceInputs, append_range, gpu_pages  # noqa: F401

OUT_ATOL = 1e-2
OUT_ARITH = 2e-3
LSE_RTOL = 1e-3
_MANT_BITS = {torch.float16: 10, torch.bfloat16: 7}


def out_tolerance(ref: np.ndarray, dtype) -> np.ndarray:
    """Per-element bound: max(1e-2, half an ulp of |ref| in dtype + 2e-3)."""
    a = np.maximum(np.abs(ref), 2.0 ** -24)
    half_ulp = np.exp2(np.floor(np.log2(a)) - _MANT_BITS[dtype] - 1)
    return np.maximum(OUT_ATOL, half_ulp + OUT_ARITH)


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def run_oracle(w, rows=None, pool=None):
    """The oracle on workload w (rows: global query tokens to evaluate, all
    when None). pool: the page pool of a paged workload as
    pages_from_logical(w) returns it, when the caller has built it already."""
    if w.kind == "mla":
        from workloads import mla_pages_from_logical
        if pool is None:
            pool = mla_pages_from_logical(w)
        return oracle.mla_paged_attn(w.q, w.q_indptr, pool, w.page_indptr, w.page_values,
                                     w.length_info, w.causal, w.sm_scale, w.d_latent, rows=rows)
    if w.kind == "ragged":
        return oracle.ragged_prefill(w.q, w.q_indptr, w.k, w.v, w.kv_indptr, w.valid_len,
                                     w.pad_mode, w.causal, w.sm_scale, rows=rows)
    if w.kind == "tree":
        return oracle.tree_attn(w.q, w.q_indptr, w.k, w.v, w.kv_indptr, w.q_rope_position,
                                w.mn_indptr, w.tree_mask, w.rotary_mode, w.rope_scale,
                                w.rope_theta, w.sm_scale, w.dtype, rows=rows)
    kw = dict(tree_order_indptr=w.tree_order_indptr, tree_order=w.tree_order,
              q_rope_position=w.q_rope_position, k_rope_pos_offset=w.k_rope_pos_offset,
              rotary_mode=w.rotary_mode, rope_scale=w.rope_scale, rope_theta=w.rope_theta,
              rows=rows)
    if w.store_rope_position is not None:
        kw.update(cache_rope_position=w.store_rope_position, cache_rope_indptr=w.kv_store_indptr)
    if pool is None:
        pool = pages_from_logical(w)
    return oracle.paged_attn(w.q, w.q_indptr, pool, w.page_indptr, w.page_values,
                             w.length_info, w.sliding_window, w.causal, w.sm_scale, w.dtype, **kw)


def sample_rows(w, per_seq: int = 4, seed: int = 0) -> np.ndarray:
    """First, last and random query tokens of every sequence."""
    rng = np.random.default_rng(seed)
    rows = []
    for b in range(w.batch):
        q0, q1 = int(w.q_indptr[b]), int(w.q_indptr[b + 1])
        if q1 == q0:
            continue
        pick = {q0, q1 - 1}
        pick.update(rng.integers(q0, q1, size=max(per_seq - 2, 0)).tolist())
        rows.extend(sorted(pick))
    return np.array(rows, dtype=np.int64)


def compare(out_gpu, lse_gpu, out_ref, lse_ref, rows=None, label=""):
    """Assert the GPU result matches the oracle on ``rows`` (all rows if None).
    Returns (max |d out|, max relative |d lse|)."""
    dtype = out_gpu.dtype
    og = out_gpu.detach().float().cpu().numpy().astype(np.float64)
    lg = lse_gpu.detach().float().cpu().numpy().astype(np.float64)
    if rows is not None:
        og, lg, out_ref, lse_ref = og[rows], lg[rows], out_ref[rows], lse_ref[rows]
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lg), empty), "%s: rows with no visible key differ" % label
    assert np.all(og[empty] == 0), "%s: empty rows must be 0" % label
    ne = ~empty
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg[ne])), "%s: non-finite output" % label
    err = np.abs(og - out_ref)
    d_out = float(np.max(err)) if og.size else 0.0
    d_lse = float(np.max(np.abs(lg[ne] - lse_ref[ne]) / np.maximum(1.0, np.abs(lse_ref[ne])))) if ne.any() else 0.0
    if og.size:
        over = err > out_tolerance(out_ref, dtype)
        if over.any():
            i = np.unravel_index(np.argmax(np.where(over, err, -1)), err.shape)
            raise AssertionError("%s: |d out| = %.3g at %s (ref %.4g) exceeds its bound (%d elements)"
                                 % (label, err[i], i, out_ref[i], int(over.sum())))
    assert d_lse <= LSE_RTOL, "%s: max rel |d lse| = %.3g > %g" % (label, d_lse, LSE_RTOL)
    return d_out, d_lse
