"""Helpers shared by the GPU parity tests: run a workload through the HIP
library (via the C ABI binding) and through the CPU oracle, and compare.

Tolerances (fp16/bf16 outputs against the float64 oracle):
  |out_gpu - out_ref| <= max(1e-2, half an ulp of |out_ref| in the dtype
    + 2e-3 + 2 u sigma) per element. Storing a correct result rounds it by up
    to half an ulp (bf16: 0.0078 for |out| in [2, 4), 0.0156 in [4, 8)). The
    kernels round the softmax weights P to the MFMA input type (relative
    error at most u = 2^-8 in bf16, 2^-11 in fp16) and divide by the sum of
    the rounded weights, which moves an output by at most
    2 u sum_j w_j |v_j - out| <= 2 u sigma, sigma being the standard
    deviation of v under the row's attention weights (the oracle reports it);
    2e-3 covers the rest (float32 accumulation, rotated inputs one storage
    ulp apart). Where the oracle gives no sigma the bound is
    max(1e-2, half an ulp + 2e-3).
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


def out_tolerance(ref: np.ndarray, dtype, spread=None) -> np.ndarray:
    """Per-element bound on |out_gpu - out_ref| (see the module docstring);
    spread: the oracle's standard deviation of v under the attention
    weights, shaped like ref, or None."""
    a = np.maximum(np.abs(ref), 2.0 ** -24)
    half_ulp = np.exp2(np.floor(np.log2(a)) - _MANT_BITS[dtype] - 1)
    bound = half_ulp + OUT_ARITH
    if spread is not None:
        u = 2.0 ** -(_MANT_BITS[dtype] + 1)      # unit roundoff of the MFMA input type
        bound = bound + 2.0 * u * np.nan_to_num(np.asarray(spread, dtype=np.float64))
    return np.maximum(OUT_ATOL, bound)


class OracleOut(np.ndarray):
    """The oracle's out array, carrying the per-element spread (standard
    deviation of v under the attention weights) that the tolerance uses.
    Arrays derived from it (slices, arithmetic) carry none."""

    def __new__(cls, out, spread):
        obj = np.asarray(out).view(cls)
        obj.spread = spread
        return obj

    def __array_finalize__(self, obj):
        self.spread = None


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def run_oracle(w, rows=None, pool=None, spread: bool = True):
    """The oracle on workload w (rows: global query tokens to evaluate, all
    when None). pool: the page pool of a paged workload as
    pages_from_logical(w) returns it, when the caller has built it already.
    Returns (out, lse); with spread, out is an OracleOut carrying the spread
    of v that the tolerance needs."""
    d_out = w.d_latent if w.kind == "mla" else w.d
    sp = np.full((w.total_q, w.h_q, d_out), np.nan) if spread else None
    extra = {} if sp is None else {"spread": sp}
    if w.kind == "mla":
        from workloads import mla_pages_from_logical
        if pool is None:
            pool = mla_pages_from_logical(w)
        out, lse = oracle.mla_paged_attn(w.q, w.q_indptr, pool, w.page_indptr, w.page_values,
                                         w.length_info, w.causal, w.sm_scale, w.d_latent, rows=rows,
                                         **extra)
    elif w.kind == "ragged":
        out, lse = oracle.ragged_prefill(w.q, w.q_indptr, w.k, w.v, w.kv_indptr, w.valid_len,
                                         w.pad_mode, w.causal, w.sm_scale, rows=rows, **extra)
    elif w.kind == "tree":
        out, lse = oracle.tree_attn(w.q, w.q_indptr, w.k, w.v, w.kv_indptr, w.q_rope_position,
                                    w.mn_indptr, w.tree_mask, w.rotary_mode, w.rope_scale,
                                    w.rope_theta, w.sm_scale, w.dtype, rows=rows, **extra)
    else:
        kw = dict(tree_order_indptr=w.tree_order_indptr, tree_order=w.tree_order,
                  q_rope_position=w.q_rope_position, k_rope_pos_offset=w.k_rope_pos_offset,
                  rotary_mode=w.rotary_mode, rope_scale=w.rope_scale, rope_theta=w.rope_theta,
                  rows=rows, **extra)
        if w.store_rope_position is not None:
            kw.update(cache_rope_position=w.store_rope_position, cache_rope_indptr=w.kv_store_indptr)
        if pool is None:
            pool = pages_from_logical(w)
        out, lse = oracle.paged_attn(w.q, w.q_indptr, pool, w.page_indptr, w.page_values,
                                     w.length_info, w.sliding_window, w.causal, w.sm_scale, w.dtype, **kw)
    return (out if sp is None else OracleOut(out, sp)), lse


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
    spread = getattr(out_ref, "spread", None)
    out_ref = np.asarray(out_ref)
    og = out_gpu.detach().float().cpu().numpy().astype(np.float64)
    lg = lse_gpu.detach().float().cpu().numpy().astype(np.float64)
    if rows is not None:
        og, lg, out_ref, lse_ref = og[rows], lg[rows], out_ref[rows], lse_ref[rows]
        spread = None if spread is None else spread[rows]
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lg), empty), "%s: rows with no visible key differ" % label
    assert np.all(og[empty] == 0), "%s: empty rows must be 0" % label
    ne = ~empty
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg[ne])), "%s: non-finite output" % label
    err = np.abs(og - out_ref)
    d_out = float(np.max(err)) if og.size else 0.0
    d_lse = float(np.max(np.abs(lg[ne] - lse_ref[ne]) / np.maximum(1.0, np.abs(lse_ref[ne])))) if ne.any() else 0.0
    if og.size:
        over = err > out_tolerance(out_ref, dtype, spread)
        if over.any():
            i = np.unravel_index(np.argmax(np.where(over, err, -1)), err.shape)
            raise AssertionError("%s: |d out| = %.3g at %s (ref %.4g) exceeds its bound (%d elements)"
                                 % (label, err[i], i, out_ref[i], int(over.sum())))
    assert d_lse <= LSE_RTOL, "%s: max rel |d lse| = %.3g > %g" % (label, d_lse, LSE_RTOL)
    return d_out, d_lse
